// launch_stubs.cpp — host-only stand-ins for the kernel launchers and the one
// HIP runtime call of fa_api.cpp, so that the C ABI (argument validation and
// packing) can be built with g++ and the address / undefined-behaviour
// sanitizers and run without a GPU. Each stub records the arguments it was
// handed; nothing is launched and no memory is touched.
#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {

// What the last stub saw, for the driver's checks.
FwdArgs g_last_fwd{};
BwdArgs g_last_bwd{};
int g_last_head_dim = 0;
int g_launches = 0;
float g_noalloc_scratch[16];

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool, bool, bool, hipStream_t) {
  g_last_fwd = a;
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool, bool, bool, bool, bool, hipStream_t) {
  g_last_bwd = a;
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_varlen(const FwdArgs& a, int head_dim, bool, bool, hipStream_t) {
  g_last_fwd = a;
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_persistent(const FwdArgs& a, int head_dim, bool, bool, hipStream_t) {
  g_last_fwd = a;
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quantize_fp8(const void*, void*, float*, const signed char*, int, int, int head_dim, hipStream_t) {
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quantize_vt_fp8(const void*, void*, float*, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const FwdArgs& a, int, bool, bool, hipStream_t) {
  g_last_fwd = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd_varlen(const BwdArgs& a, int head_dim, bool, bool, bool, bool, hipStream_t) {
  g_last_bwd = a;
  g_last_head_dim = head_dim;
  ++g_launches;
  return hipSuccess;
}
hipError_t bwd_noalloc_scratch(float** dvec) {
  *dvec = g_noalloc_scratch;
  return hipSuccess;
}

}  // namespace fa

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
