// abi_driver.cpp — drives every entry point of the C ABI (fa_api.cpp, built
// with launch_stubs.cpp instead of the kernels) through valid and invalid
// arguments: extreme sizes near the 32-bit limits, every error code, NULL and
// misaligned pointers, non-finite scales. Built with the host address and
// undefined-behaviour sanitizers, it must finish without a sanitizer report
// and with every expectation met; it prints "abi driver ok" and exits 0.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "fa.h"
#include "fa_launch.h"

namespace fa {
extern FwdArgs g_last_fwd;
extern BwdArgs g_last_bwd;
extern int g_launches;
}  // namespace fa

static int g_failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED: %s (line %d)\n", #cond, __LINE__); \
      ++g_failures;                                                    \
    }                                                                  \
  } while (0)

// fake, 16-byte aligned device addresses, never dereferenced
static void* const P = reinterpret_cast<void*>(uintptr_t{0x10000});
static void* const MIS = reinterpret_cast<void*>(uintptr_t{0x10008});
static const int* const CU = reinterpret_cast<const int*>(uintptr_t{0x20000});

static int fwd(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int in_dt, int out_dt,
               void* q = P) {
  return fa_fwd(q, P, P, P, (float*)P, B, Hq, Hkv, Nq, Nk, d, scale, causal, in_dt, out_dt, nullptr);
}

static int bwd(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int prec, float* ws = (float*)P) {
  return fa_bwd(P, P, P, P, (const float*)P, P, (float*)P, P, P, ws, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                FA_DTYPE_BF16, FA_DTYPE_F32, FA_DTYPE_F32, prec, nullptr);
}

int main() {
  const float inf = std::numeric_limits<float>::infinity();
  const float nan = std::numeric_limits<float>::quiet_NaN();

  // valid calls reach the launcher with the right packing
  int n0 = fa::g_launches;
  EXPECT(fwd(2, 8, 2, 300, 300, 128, 0.125f, 1, FA_DTYPE_BF16, FA_DTYPE_F32) == FA_OK);
  EXPECT(fa::g_launches == n0 + 1);
  EXPECT(fa::g_last_fwd.G == 4 && fa::g_last_fwd.B == 2 && fa::g_last_fwd.Nq == 300);
  EXPECT(fa::g_last_fwd.c > 0.0f && fa::g_last_fwd.neg == 0);
  EXPECT(fwd(1, 1, 1, 1, 1, 64, -0.5f, 0, FA_DTYPE_F32, FA_DTYPE_BF16) == FA_OK);
  EXPECT(fa::g_last_fwd.neg == 1);
  EXPECT(fwd(1, 1, 1, 1, 1, 64, 0.0f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_OK);
  EXPECT(fa::g_last_fwd.c > 0.0f);  // zero scale enters as the smallest normal multiplier
  // largest sizes the checks let through (no overflow in the checks or the packing)
  EXPECT(fwd(1, 1, 1, (1 << 24) - 1, (1 << 24) - 1, 128, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_OK);
  EXPECT(fwd(1, 1, 1, (1 << 25) - 1, 5, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_OK);
  EXPECT(fwd(2097151, 1, 1, 1, 1, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_OK);

  // every error code, before any launch
  n0 = fa::g_launches;
  EXPECT(fwd(1, 1, 1, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16, MIS) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(0, 1, 1, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(INT_MIN, 1, 1, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 3, 2, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 64, nan, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 64, -inf, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 64, 0.1f, 2, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 64, 0.1f, 0, 7, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(1, 1, 1, 16, 16, 96, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_UNSUPPORTED);
  EXPECT(fwd(1, 1, 1, 16, 17, 64, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_UNSUPPORTED);
  EXPECT(fwd(1, 1, 1, INT_MAX, INT_MAX, 128, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(INT_MAX, INT_MAX, 1, 16, 16, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fwd(2097152, 1, 1, 1, 1, 64, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16) == FA_ERR_INVALID_ARGUMENT);

  // backward: both precisions, the atomic scheme, the workspace
  EXPECT(bwd(4, 16, 16, 4096, 4096, 128, 0.088f, 1, FA_PRECISION_BF16) == FA_OK);
  EXPECT(fa::g_last_bwd.dvec == (float*)P && fa::g_last_bwd.G == 1);
  EXPECT(bwd(1, 8, 1, 512, 512, 128, 0.088f, 1, FA_PRECISION_HILO) == FA_OK);
  EXPECT(bwd(1, 8, 1, 512, 512, 128, 0.088f, 1, 2) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(bwd(1, 8, 1, 512, 512, 128, 0.088f, 1, FA_PRECISION_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd_atomic(P, P, P, P, (const float*)P, P, (float*)P, P, P, (float*)P, 1, 2, 1, 16, 16, 64, 0.1f, 0,
                       FA_DTYPE_BF16, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_PRECISION_HILO, nullptr) == FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd(P, P, P, P, (const float*)P, P, (float*)P, P, P, (float*)P, 1, 2, 1, 16, 16, 64, 0.1f, 0,
                FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_PRECISION_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd_workspace_bytes(4, 16, 4096) == (size_t)4 * 4 * 16 * 4096);
  EXPECT(fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX) == (size_t)4 * INT_MAX * (size_t)INT_MAX * INT_MAX);
  EXPECT(fa_bwd_workspace_bytes(-1, 1, 1) == 0);

  // no-allocation backward: the row limit, checked before the scratch lookup
  EXPECT(fa_bwd_noalloc(P, P, P, P, (const float*)P, P, (float*)P, P, P, 4, 16, 16, 4096, 4096, 128, 0.088f, 1,
                        FA_DTYPE_BF16, FA_DTYPE_F32, FA_DTYPE_F32, FA_PRECISION_BF16, nullptr) == FA_OK);
  EXPECT(fa::g_last_bwd.dvec != nullptr && fa::g_last_bwd.dvec != (float*)P);
  EXPECT(fa_bwd_noalloc(P, P, P, P, (const float*)P, P, (float*)P, P, P, 1, 1, 1, FA_BWD_NOALLOC_MAX_ROWS,
                        FA_BWD_NOALLOC_MAX_ROWS, 64, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_F32, FA_DTYPE_F32,
                        FA_PRECISION_BF16, nullptr) == FA_OK);
  EXPECT(fa_bwd_noalloc(P, P, P, P, (const float*)P, P, (float*)P, P, P, 1, 1, 1, FA_BWD_NOALLOC_MAX_ROWS + 1,
                        FA_BWD_NOALLOC_MAX_ROWS + 1, 64, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_F32, FA_DTYPE_F32,
                        FA_PRECISION_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd_noalloc(P, P, P, P, (const float*)P, P, (float*)P, P, P, 2047, 2047, 1, 2047, 2047, 64, 0.1f, 0,
                        FA_DTYPE_BF16, FA_DTYPE_F32, FA_DTYPE_F32, FA_PRECISION_BF16, nullptr) ==
         FA_ERR_INVALID_ARGUMENT);

  // variable-length entry points
  EXPECT(fa_fwd_varlen(P, P, P, P, (float*)P, CU, CU, 3, 100, 100, 250, 250, 4, 2, 128, 0.1f, 1, FA_DTYPE_BF16,
                       FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa::g_last_fwd.total_q == 250 && fa::g_last_fwd.cu_q == CU);
  EXPECT(fa_fwd_varlen(P, P, P, P, (float*)P, CU, CU, 3, 0, 0, 0, 0, 4, 2, 128, 0.1f, 0, FA_DTYPE_BF16,
                       FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_fwd_varlen(P, P, P, P, (float*)P, CU, CU, 3, 251, 100, 250, 250, 4, 2, 128, 0.1f, 0, FA_DTYPE_BF16,
                       FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd_varlen(P, P, P, P, (const float*)P, P, (float*)P, P, P, (float*)P, CU, CU, 3, 100, 100, 250, 250, 4,
                       2, 128, 0.1f, 1, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_PRECISION_HILO,
                       nullptr) == FA_OK);
  EXPECT(fa_bwd_varlen(P, P, P, P, (const float*)P, P, (float*)P, P, P, (float*)P, CU, CU, 3, 100, 100, INT_MAX,
                       INT_MAX, 4, 2, 128, 0.1f, 0, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_PRECISION_BF16,
                       nullptr) == FA_ERR_INVALID_ARGUMENT);

  // FP8, persistent, sizes and strings
  EXPECT(fa_quantize_fp8(P, P, (float*)P, nullptr, 2, 4, 1000, 128, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_quantize_fp8(P, P, (float*)P, nullptr, 2, 4, INT_MAX, 128, FA_DTYPE_BF16, nullptr) ==
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fp8_scales_count(INT_MAX, INT_MAX, INT_MAX) > 0);
  EXPECT(fa_fwd_fp8(P, (const float*)P, P, (const float*)P, P, P, (float*)P, 1, 2, 1, 64, 64, 64, 0.1f, 0,
                    FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_fwd_fp8(P, (const float*)P, P, (const float*)P, P, P, (float*)P, 1, 2, 1, 64, 64, 96, 0.1f, 0,
                    FA_DTYPE_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  EXPECT(fa_quantize_vt_fp8(P, P, (float*)P, 2, 4, 1000, 64, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_quantize_vt_fp8(P, P, (float*)P, 2, 4, INT_MAX, 128, FA_DTYPE_BF16, nullptr) ==
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fp8_vt_bytes(INT_MAX, INT_MAX, INT_MAX, 128) > 0);
  EXPECT(fa_fwd_fp8_pv(P, (const float*)P, P, (const float*)P, P, (const float*)P, P, (float*)P, 1, 2, 1, 64, 64,
                       128, 0.1f, 1, FA_DTYPE_F32, nullptr) == FA_OK);
  EXPECT(fa_fwd_fp8_pv(P, (const float*)P, P, (const float*)P, P, nullptr, P, (float*)P, 1, 2, 1, 64, 64, 128, 0.1f,
                       1, FA_DTYPE_F32, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_fp8_quantize_q(P, nullptr, P, (const float*)P, P, nullptr, P, (float*)P, 1, 2, 1, 64, 64, 128, 0.1f,
                               1, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_fwd_fp8_quantize_q(P, (const signed char*)P, P, (const float*)P, P, (const float*)P, P, (float*)P, 1, 2,
                               1, 64, 64, 64, -0.1f, 0, FA_DTYPE_F32, nullptr) == FA_OK);
  EXPECT(fa_fwd_fp8_quantize_q(P, nullptr, P, nullptr, P, nullptr, P, (float*)P, 1, 2, 1, 64, 64, 128, 0.1f, 1,
                               FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_fp8_quantize_q(P, nullptr, P, (const float*)P, P, (const float*)(uintptr_t{0x10002}), P, (float*)P, 1,
                               2, 1, 64, 64, 128, 0.1f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_fp8_quantize_q(P, nullptr, P, (const float*)P, P, nullptr, P, (float*)P, 1, 2, 1, 64, 64, 96, 0.1f,
                               1, FA_DTYPE_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_persistent(P, P, P, P, (float*)P, (int*)P, 1, 2, 1, 64, 64, 128, 0.1f, 1, FA_DTYPE_BF16,
                           FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_fwd_persistent(P, P, P, P, (float*)P, (int*)(uintptr_t{0x10002}), 1, 2, 1, 64, 64, 128, 0.1f, 1,
                           FA_DTYPE_BF16, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARGUMENT);
  for (int st = -1; st <= 4; ++st) EXPECT(fa_status_string(st) != nullptr);
  EXPECT(fa_last_error() != nullptr);
  EXPECT(fa_version() == 2);

  if (g_failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi driver ok\n");
  return 0;
}
