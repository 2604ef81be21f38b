// fa_launch.h — internal interface between the C ABI (fa_api.cpp) and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, G, Nq, Nk;
  float c;        // |scale| * log2(e): scores are scaled in base 2
  int neg;        // scale < 0: Q is negated as it is loaded
  int n_q_tiles;  // filled in by the launcher
  // Packed variable-length batch (fa_fwd_varlen): per-sequence cumulative
  // row offsets [B + 1]; Nq / Nk then hold the maximum sequence lengths and
  // total_q / total_k the packed row counts. Unused by fa_fwd.
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // FP8 forward (fa_fwd_fp8): q and k hold e4m3 codes; the power-of-two scale
  // of each 64-row block, [B][Hq][ceil(Nq/64)] and [B][Hkv][ceil(Nk/64)].
  // q_scales null (fa_fwd_fp8_quantize_q): q is bf16, quantized in the
  // kernel with the random signs q_signs [d] (null: no transform).
  const float* q_scales;
  const float* k_scales;
  const signed char* q_signs;
  // FP8 P V (fa_fwd_fp8_pv): v holds the transposed codes of
  // fa_quantize_vt_fp8 and v_scales their block scales [B][Hkv][ceil(Nk/64)];
  // null for the bf16 V of fa_fwd_fp8.
  const float* v_scales;
  // Persistent forward (fa_fwd_persistent): 9 work-queue counters, zero on
  // entry and left zero on exit.
  int* sched;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  void* dk;
  void* dv;
  float* dvec;  // D = rowsum(dO o O), fp32 [B][Hq][Nq]
  int o_f32;    // O is fp32 (else bf16)
  int B, Hq, Hkv, G, Nq, Nk;
  float scale;
  float c;  // scale * log2(e)
  // Packed variable-length batch (fa_bwd_varlen), as in FwdArgs.
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
};

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool in_f32, bool causal, bool out_f32, hipStream_t s);
// hilo: P and dS enter the gradient products as bf16 pairs hi + lo
// (FA_PRECISION_HILO); the atomic scheme does not take it.
hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool causal, bool o_f32, bool grad_f32, bool atomic_dq,
                      bool hilo, hipStream_t s);
hipError_t launch_fwd_varlen(const FwdArgs& a, int head_dim, bool causal, bool out_f32, hipStream_t s);
hipError_t launch_fwd_persistent(const FwdArgs& a, int head_dim, bool causal, bool out_f32, hipStream_t s);
hipError_t launch_quantize_fp8(const void* x, void* codes, float* scales, const signed char* signs, int heads,
                               int N, int head_dim, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs& a, int head_dim, bool causal, bool out_f32, hipStream_t s);
hipError_t launch_quantize_vt_fp8(const void* v, void* codes, float* scales, int heads, int N, int head_dim,
                                  hipStream_t s);
// fa_bwd_noalloc keeps D in a static device array of this many fp32 rows
// (16 MiB per device); bwd_noalloc_scratch returns its device address on the
// current device (looked up once per device, with hipGetSymbolAddress).
constexpr long long kBwdNoallocMaxRows = 1LL << 22;
hipError_t bwd_noalloc_scratch(float** dvec);

hipError_t launch_bwd_varlen(const BwdArgs& a, int head_dim, bool causal, bool o_f32, bool grad_f32, bool hilo,
                             hipStream_t s);

}  // namespace fa
