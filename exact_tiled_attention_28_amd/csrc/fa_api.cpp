// fa_api.cpp — the C ABI declared in include/fa.h: validate on the host,
// pick the kernel instantiation, launch on the caller's stream, return.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/fa.h"
#include "fa_args.h"
#include "fa_launch.h"

static_assert(FA_BWD_NOALLOC_MAX_ROWS == fa::kBwdNoallocMaxRows, "fa.h and the scratch array must agree");

namespace {

thread_local std::string g_last_error;

int fail(int rc, const std::string& msg) {
  g_last_error = msg;
  return rc;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Multiplier of the raw scores in the bf16/fp32 forward kernels' exp2
// arguments, |scale| log2(e) (a negative scale negates Q instead). A zero
// scale is raised to the smallest normal float: the kernels set masked
// scores to -inf and rely on -inf * c staying -inf (0 * -inf would be NaN),
// so that exp2 yields 0 with no per-element test. Scaled scores of any
// realistic size are then far below fp32 resolution next to 0 and 1, so
// every visible key gets probability exactly 1 before normalisation, as
// with a zero scale.
float fwd_exp2_mult(float scale) { return std::fmax(std::fabs(scale) * 1.4426950408889634f, FLT_MIN); }

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int n_q_heads,
           int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal, int in_dtype,
           int out_dtype, void* stream) {
  std::string err;
  const fa::Shape s{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim};
  if (int rc = fa::check_fwd(q, k, v, o, lse, s, scale, causal, in_dtype, out_dtype, err)) return fail(rc, err);
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.c = fwd_exp2_mult(scale);
  a.neg = scale < 0.0f;
  hipError_t e = fa::launch_fwd(a, head_dim, in_dtype == FA_DTYPE_F32, causal != 0, out_dtype == FA_DTYPE_F32,
                                (hipStream_t)stream);
  return hip_status(e, "fa_fwd launch");
}

int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int* sched, int batch,
                      int n_q_heads, int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim, float scale,
                      int causal, int in_dtype, int out_dtype, void* stream) {
  std::string err;
  const fa::Shape s{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim};
  if (int rc = fa::check_fwd(q, k, v, o, lse, s, scale, causal, in_dtype, out_dtype, err)) return fail(rc, err);
  if (sched == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "sched is NULL");
  if (reinterpret_cast<uintptr_t>(sched) & 3u) return fail(FA_ERR_INVALID_ARGUMENT, "sched is not 4-byte aligned");
  if (in_dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the persistent forward takes bf16 q, k, v");
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.c = fwd_exp2_mult(scale);
  a.neg = scale < 0.0f;
  a.sched = sched;
  hipError_t e = fa::launch_fwd_persistent(a, head_dim, causal != 0, out_dtype == FA_DTYPE_F32, (hipStream_t)stream);
  return hip_status(e, "fa_fwd_persistent launch");
}

size_t fa_fwd_persistent_sched_bytes(void) { return 9 * sizeof(int); }

}  // extern "C"

static int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, float* dq, void* dk, void* dv, float* workspace, int batch, int n_q_heads,
                      int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                      int in_dtype, int o_dtype, int grad_dtype, int precision, void* stream, bool atomic_dq,
                      const char* name) {
  std::string err;
  const fa::Shape s{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim};
  if (int rc = fa::check_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, s, scale, causal, in_dtype, o_dtype,
                             grad_dtype, err))
    return fail(rc, err);
  if (int rc = fa::check_precision(precision, atomic_dq, err)) return fail(rc, err);
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dvec = workspace;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  hipError_t e = fa::launch_bwd(a, head_dim, causal != 0, o_dtype == FA_DTYPE_F32, grad_dtype == FA_DTYPE_F32,
                                atomic_dq, precision == FA_PRECISION_HILO, (hipStream_t)stream);
  return hip_status(e, name);
}

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           float* dq, void* dk, void* dv, float* workspace, int batch, int n_q_heads, int n_kv_heads, int seqlen_q,
           int seqlen_k, int head_dim, float scale, int causal, int in_dtype, int o_dtype, int grad_dtype,
           int precision, void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
                    head_dim, scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream, false,
                    "fa_bwd launch");
}

int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  float* dq, void* dk, void* dv, float* workspace, int batch, int n_q_heads, int n_kv_heads,
                  int seqlen_q, int seqlen_k, int head_dim, float scale, int causal, int in_dtype, int o_dtype,
                  int grad_dtype, int precision, void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k,
                    head_dim, scale, causal, in_dtype, o_dtype, grad_dtype, precision, stream, true,
                    "fa_bwd_atomic launch");
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   float* dq, void* dk, void* dv, int batch, int n_q_heads, int n_kv_heads, int seqlen_q,
                   int seqlen_k, int head_dim, float scale, int causal, int in_dtype, int o_dtype, int grad_dtype,
                   int precision, void* stream) {
  std::string err;
  const fa::Shape s{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim};
  if (int rc = fa::check_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, s, scale, causal, in_dtype, o_dtype,
                             grad_dtype, err, false))
    return fail(rc, err);
  if (int rc = fa::check_precision(precision, false, err)) return fail(rc, err);
  const long long rows = (long long)batch * n_q_heads * seqlen_q;
  if (rows > fa::kBwdNoallocMaxRows)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd_noalloc: batch * n_q_heads * seqlen_q = " + std::to_string(rows) +
                                             " exceeds its scratch of " + std::to_string(fa::kBwdNoallocMaxRows) +
                                             " rows (FA_BWD_NOALLOC_MAX_ROWS)");
  float* dvec = nullptr;
  if (hipError_t e = fa::bwd_noalloc_scratch(&dvec); e != hipSuccess)
    return hip_status(e, "fa_bwd_noalloc scratch lookup");
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dvec = dvec;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  hipError_t e = fa::launch_bwd(a, head_dim, causal != 0, o_dtype == FA_DTYPE_F32, grad_dtype == FA_DTYPE_F32, false,
                                precision == FA_PRECISION_HILO, (hipStream_t)stream);
  return hip_status(e, "fa_bwd_noalloc launch");
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int n_q_heads, int n_kv_heads, int head_dim, float scale, int causal, int in_dtype, int out_dtype,
                  void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_ptr(q, "q", err)) || (rc = fa::check_ptr(k, "k", err)) || (rc = fa::check_ptr(v, "v", err)) ||
      (rc = fa::check_ptr(o, "o", err)) || (rc = fa::check_ptr(lse, "lse", err)))
    return fail(rc, err);
  if (!fa::valid_dtype(in_dtype) || !fa::valid_dtype(out_dtype))
    return fail(FA_ERR_INVALID_ARGUMENT, "in_dtype and out_dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16");
  const fa::VarlenShape s{batch, max_seqlen_q, max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, head_dim};
  if ((rc = fa::check_varlen(cu_seqlens_q, cu_seqlens_k, s, scale, causal, err))) return fail(rc, err);
  if (in_dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the variable-length forward takes bf16 q, k, v");
  if (max_seqlen_q == 0) return FA_OK;  // no query rows at all
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = max_seqlen_q;
  a.Nk = max_seqlen_k;
  a.c = fwd_exp2_mult(scale);
  a.neg = scale < 0.0f;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  hipError_t e = fa::launch_fwd_varlen(a, head_dim, causal != 0, out_dtype == FA_DTYPE_F32, (hipStream_t)stream);
  return hip_status(e, "fa_fwd_varlen launch");
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  float* dq, void* dk, void* dv, float* workspace, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int n_q_heads,
                  int n_kv_heads, int head_dim, float scale, int causal, int in_dtype, int o_dtype, int grad_dtype,
                  int precision, void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_ptr(q, "q", err)) || (rc = fa::check_ptr(k, "k", err)) || (rc = fa::check_ptr(v, "v", err)) ||
      (rc = fa::check_ptr(o, "o", err)) || (rc = fa::check_ptr(lse, "lse", err)) ||
      (rc = fa::check_ptr(dout, "dout", err)) || (rc = fa::check_ptr(dq, "dq", err)) ||
      (rc = fa::check_ptr(dk, "dk", err)) || (rc = fa::check_ptr(dv, "dv", err)) ||
      (rc = fa::check_ptr(workspace, "workspace", err)))
    return fail(rc, err);
  if (!fa::valid_dtype(in_dtype) || !fa::valid_dtype(o_dtype) || !fa::valid_dtype(grad_dtype))
    return fail(FA_ERR_INVALID_ARGUMENT, "dtypes must be FA_DTYPE_F32 or FA_DTYPE_BF16");
  const fa::VarlenShape s{batch, max_seqlen_q, max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, head_dim};
  if ((rc = fa::check_varlen(cu_seqlens_q, cu_seqlens_k, s, scale, causal, err))) return fail(rc, err);
  if (in_dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the backward pass takes bf16 q, k, v, dout");
  if ((rc = fa::check_precision(precision, false, err))) return fail(rc, err);
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dvec = workspace;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = max_seqlen_q;
  a.Nk = max_seqlen_k;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  hipError_t e = fa::launch_bwd_varlen(a, head_dim, causal != 0, o_dtype == FA_DTYPE_F32, grad_dtype == FA_DTYPE_F32,
                                       precision == FA_PRECISION_HILO, (hipStream_t)stream);
  return hip_status(e, "fa_bwd_varlen launch");
}

int fa_quantize_fp8(const void* x, void* codes, float* block_scales, const signed char* signs, int batch,
                    int n_heads, int seqlen, int head_dim, int in_dtype, void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_ptr(x, "x", err)) || (rc = fa::check_ptr(codes, "codes", err))) return fail(rc, err);
  if (block_scales == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "block_scales is NULL");
  if (reinterpret_cast<uintptr_t>(block_scales) & 3u)
    return fail(FA_ERR_INVALID_ARGUMENT, "block_scales is not 4-byte aligned");
  if (batch < 1 || n_heads < 1 || seqlen < 1) return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (!fa::valid_dtype(in_dtype)) return fail(FA_ERR_INVALID_ARGUMENT, "in_dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16");
  if (in_dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "fa_quantize_fp8 takes bf16 input");
  if (head_dim != 64 && head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) +
                                                     " unsupported (64 or 128)");
  if ((long long)seqlen * head_dim >= (1LL << 31)) return fail(FA_ERR_INVALID_ARGUMENT, "seqlen * head_dim must be below 2^31");
  if ((long long)batch * n_heads * (((long long)seqlen + 63) / 64) >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARGUMENT, "batch * n_heads * blocks too large");
  hipError_t e = fa::launch_quantize_fp8(x, codes, block_scales, signs, batch * n_heads, seqlen, head_dim,
                                         (hipStream_t)stream);
  return hip_status(e, "fa_quantize_fp8 launch");
}

int fa_fwd_fp8(const void* q_codes, const float* q_scales, const void* k_codes, const float* k_scales, const void* v,
               void* o, float* lse, int batch, int n_q_heads, int n_kv_heads, int seqlen_q, int seqlen_k,
               int head_dim, float scale, int causal, int out_dtype, void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_fwd(q_codes, k_codes, v, o, lse,
                          fa::Shape{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim}, scale, causal,
                          FA_DTYPE_BF16, out_dtype, err)))
    return fail(rc, err);
  if (q_scales == nullptr || k_scales == nullptr)
    return fail(FA_ERR_INVALID_ARGUMENT, q_scales == nullptr ? "q_scales is NULL" : "k_scales is NULL");
  if ((reinterpret_cast<uintptr_t>(q_scales) & 3u) || (reinterpret_cast<uintptr_t>(k_scales) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "q_scales / k_scales must be 4-byte aligned");

  fa::FwdArgs a{};
  a.q = q_codes;
  a.k = k_codes;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.c = std::fabs(scale) * 1.4426950408889634f;
  a.neg = scale < 0.0f;
  a.q_scales = q_scales;
  a.k_scales = k_scales;
  hipError_t e = fa::launch_fwd_fp8(a, head_dim, causal != 0, out_dtype == FA_DTYPE_F32, (hipStream_t)stream);
  return hip_status(e, "fa_fwd_fp8 launch");
}

int fa_quantize_vt_fp8(const void* v, void* vt_codes, float* block_scales, int batch, int n_heads, int seqlen,
                       int head_dim, int in_dtype, void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_ptr(v, "v", err)) || (rc = fa::check_ptr(vt_codes, "vt_codes", err))) return fail(rc, err);
  if (block_scales == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "block_scales is NULL");
  if (reinterpret_cast<uintptr_t>(block_scales) & 3u)
    return fail(FA_ERR_INVALID_ARGUMENT, "block_scales is not 4-byte aligned");
  if (batch < 1 || n_heads < 1 || seqlen < 1) return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (!fa::valid_dtype(in_dtype)) return fail(FA_ERR_INVALID_ARGUMENT, "in_dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16");
  if (in_dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "fa_quantize_vt_fp8 takes bf16 input");
  if (head_dim != 64 && head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) +
                                                     " unsupported (64 or 128)");
  if ((long long)seqlen * head_dim >= (1LL << 31)) return fail(FA_ERR_INVALID_ARGUMENT, "seqlen * head_dim must be below 2^31");
  if ((long long)batch * n_heads * (((long long)seqlen + 63) / 64) >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARGUMENT, "batch * n_heads * blocks too large");
  hipError_t e = fa::launch_quantize_vt_fp8(v, vt_codes, block_scales, batch * n_heads, seqlen, head_dim,
                                            (hipStream_t)stream);
  return hip_status(e, "fa_quantize_vt_fp8 launch");
}

size_t fa_fp8_vt_bytes(int batch, int n_heads, int seqlen, int head_dim) {
  if (batch <= 0 || n_heads <= 0 || seqlen <= 0 || head_dim <= 0) return 0;
  return (size_t)batch * (size_t)n_heads * (((size_t)seqlen + 63) / 64) * 64 * (size_t)head_dim;
}

int fa_fwd_fp8_pv(const void* q_codes, const float* q_scales, const void* k_codes, const float* k_scales,
                  const void* vt_codes, const float* v_scales, void* o, float* lse, int batch, int n_q_heads,
                  int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal, int out_dtype,
                  void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_fwd(q_codes, k_codes, vt_codes, o, lse,
                          fa::Shape{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim}, scale, causal,
                          FA_DTYPE_BF16, out_dtype, err)))
    return fail(rc, err);
  if (q_scales == nullptr || k_scales == nullptr || v_scales == nullptr)
    return fail(FA_ERR_INVALID_ARGUMENT, q_scales == nullptr ? "q_scales is NULL"
                                         : (k_scales == nullptr ? "k_scales is NULL" : "v_scales is NULL"));
  if ((reinterpret_cast<uintptr_t>(q_scales) & 3u) || (reinterpret_cast<uintptr_t>(k_scales) & 3u) ||
      (reinterpret_cast<uintptr_t>(v_scales) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "q_scales / k_scales / v_scales must be 4-byte aligned");
  if ((long long)batch * n_kv_heads * (((long long)seqlen_k + 63) / 64) * 64 * head_dim >= (1LL << 40))
    return fail(FA_ERR_INVALID_ARGUMENT, "vt_codes too large");
  fa::FwdArgs a{};
  a.q = q_codes;
  a.k = k_codes;
  a.v = vt_codes;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.c = std::fabs(scale) * 1.4426950408889634f;
  a.neg = scale < 0.0f;
  a.q_scales = q_scales;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  hipError_t e = fa::launch_fwd_fp8(a, head_dim, causal != 0, out_dtype == FA_DTYPE_F32, (hipStream_t)stream);
  return hip_status(e, "fa_fwd_fp8_pv launch");
}

int fa_fwd_fp8_quantize_q(const void* q, const signed char* q_signs, const void* k_codes, const float* k_scales,
                          const void* v, const float* v_scales, void* o, float* lse, int batch, int n_q_heads,
                          int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                          int out_dtype, void* stream) {
  std::string err;
  int rc;
  if ((rc = fa::check_fwd(q, k_codes, v, o, lse, fa::Shape{batch, n_q_heads, n_kv_heads, seqlen_q, seqlen_k, head_dim},
                          scale, causal, FA_DTYPE_BF16, out_dtype, err)))
    return fail(rc, err);
  if (k_scales == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "k_scales is NULL");
  if ((reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "k_scales / v_scales must be 4-byte aligned");
  if (v_scales != nullptr &&
      (long long)batch * n_kv_heads * (((long long)seqlen_k + 63) / 64) * 64 * head_dim >= (1LL << 40))
    return fail(FA_ERR_INVALID_ARGUMENT, "vt_codes too large");
  fa::FwdArgs a{};
  a.q = q;
  a.k = k_codes;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.Nq = seqlen_q;
  a.Nk = seqlen_k;
  a.c = std::fabs(scale) * 1.4426950408889634f;
  a.neg = scale < 0.0f;
  a.q_scales = nullptr;  // Q is quantized in the kernel
  a.q_signs = q_signs;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  hipError_t e = fa::launch_fwd_fp8(a, head_dim, causal != 0, out_dtype == FA_DTYPE_F32, (hipStream_t)stream);
  return hip_status(e, "fa_fwd_fp8_quantize_q launch");
}

size_t fa_fp8_scales_count(int batch, int n_heads, int seqlen) {
  if (batch <= 0 || n_heads <= 0 || seqlen <= 0) return 0;
  return (size_t)batch * (size_t)n_heads * (((size_t)seqlen + 63) / 64);
}

size_t fa_bwd_workspace_bytes(int batch, int n_q_heads, int seqlen_q) {
  if (batch <= 0 || n_q_heads <= 0 || seqlen_q <= 0) return 0;
  return (size_t)4 * (size_t)batch * (size_t)n_q_heads * (size_t)seqlen_q;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return 2; }

}  // extern "C"
