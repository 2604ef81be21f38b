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
  int B, Hq, Hkv, G, Nq, Nk;
  float scale;
  float c;  // scale * log2(e)
};

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool in_f32, bool causal, bool out_f32, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool causal, bool o_f32, bool grad_f32, bool atomic_dq,
                      hipStream_t s);

}  // namespace fa
