// Test helper (not part of libfa): evaluates single FP8 dot products of 64
// terms on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unscaled), so that a test
// can check the accumulation property that the FP8 forward's parity bound
// rests on. One wavefront per case; case i supplies 64 A codes, 64 B codes
// and an fp32 accumulator input, and out[i] receives element (0, 0) of the
// product: sum_k decode(a_k) decode(b_k) + c. In the instruction's operand
// layout, lane 32 g (g = 0, 1) holds codes 32 g .. 32 g + 31 of row / column
// 0; all other lanes hold zeros.
#include <hip/hip_runtime.h>

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

struct ProbeCase {
  unsigned char a[64];
  unsigned char b[64];
  float c;
};

__global__ void __launch_bounds__(64) fp8_dot_kernel(const ProbeCase* __restrict__ cases, float* __restrict__ out) {
  const ProbeCase& pc = cases[blockIdx.x];
  const int lane = threadIdx.x;
  i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0}, b = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((lane & 31) == 0) {
    const int k0 = 32 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unsigned x = 0, y = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x |= (unsigned)pc.a[k0 + 4 * i + j] << (8 * j);
        y |= (unsigned)pc.b[k0 + 4 * i + j] << (8 * j);
      }
      a[i] = (int)x;
      b[i] = (int)y;
    }
  }
  f32x16 acc = {};
  if (lane == 0) acc[0] = pc.c;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
  if (lane == 0) out[blockIdx.x] = acc[0];
}

// cases: device array of n ProbeCase (132 bytes each, packed as declared);
// out: device float[n]. Returns 0 or the HIP error code of the launch.
extern "C" int fp8_dot_probe(const void* cases, float* out, int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fp8_dot_kernel, dim3((unsigned)n), dim3(64), 0, (hipStream_t)stream,
                     (const ProbeCase*)cases, out);
  return (int)hipGetLastError();
}

extern "C" int fp8_dot_probe_case_bytes(void) { return (int)sizeof(ProbeCase); }

// Converts n fp32 values (n a multiple of 4) to e4m3 codes with the pair
// conversion the FP8 forward uses for P (v_cvt_pk_fp8_f32, round to nearest
// even): four values per thread, packed into one 32-bit word as bytes 0-3.
__global__ void __launch_bounds__(256) fp8_cvt_kernel(const float* __restrict__ in, unsigned* __restrict__ out,
                                                      int nwords) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= nwords) return;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(in[4 * t], in[4 * t + 1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(in[4 * t + 2], in[4 * t + 3], w, true);
  out[t] = (unsigned)w;
}

// in: device float[n], out: device uint8[n] (n a multiple of 4). Returns 0
// or the HIP error code of the launch.
extern "C" int fp8_cvt_probe(const float* in, void* out, int n, void* stream) {
  if (n <= 0 || (n & 3)) return n == 0 ? 0 : -1;
  const int nwords = n / 4;
  hipLaunchKernelGGL(fp8_cvt_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, (hipStream_t)stream, in,
                     (unsigned*)out, nwords);
  return (int)hipGetLastError();
}
