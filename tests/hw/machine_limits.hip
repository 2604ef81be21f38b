// machine_limits.hip — in-bounds microbenchmarks of the gfx950 units the
// attention kernels lean on (measurement helper, not part of the library):
//   * the bf16 matrix core: independent v_mfma_f32_32x32x16_bf16 chains;
//   * exp next to the matrix core: per MFMA, E v_exp_f32 and 3 FMAs on
//     independent registers, to see how much vector work hides under it;
//   * LDS reads in the two operand patterns of the kernels: ds_read_b128 of
//     32 consecutive 256-byte rows at one 16-byte chunk, and ds_read_b64_tr_b16
//     of 4-row groups, both through the row-mod-16 XOR swizzle of the tiles;
//   * the shader clock: s_memtime (shader clock) against s_memrealtime (a
//     fixed 100 MHz counter) over the timed loop of block 0.
// Every kernel runs a fixed iteration count, writes one value per lane to
// `out` (so nothing is optimised away) and block 0 / thread 0 writes its four
// time stamps to `clk` with an ordinary vector store.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void stamp(uint64_t* clk, int slot) {
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[2 * slot] = t;
    clk[2 * slot + 1] = r;
  }
}

__device__ __forceinline__ bf16x8 lane_bf16x8(int lane, float s) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(s * (float)((lane * 8 + i) % 13 - 6));
  return v;
}

// Four independent accumulators per wavefront: the matrix core never waits
// on a result.
__global__ void __launch_bounds__(256) k_mfma(float* out, int iters, uint64_t* clk) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 0.01f), b = lane_bf16x8(lane + 1, 0.02f);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  stamp(clk, 1);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Per iteration: 4 MFMAs (when M) and, per MFMA, E exps and 3 FMAs on
// registers of their own (each a recurrence that stays in [0.5, 2], so the
// values neither overflow nor collapse).
template <bool M, int E>
__global__ void __launch_bounds__(256) k_exp(float* out, int iters, uint64_t* clk) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 0.01f), b = lane_bf16x8(lane + 1, 0.02f);
  f32x16 c[4] = {};
  float x[4][E > 0 ? E : 1], y[4][3];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int e = 0; e < (E > 0 ? E : 1); ++e) x[m][e] = 1.0f + 0.01f * (lane + e + m);
#pragma unroll
    for (int v = 0; v < 3; ++v) y[m][v] = 1.0f + 0.02f * (lane + v + m);
  }
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (M) c[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[m], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < E; ++e) x[m][e] = __builtin_amdgcn_exp2f(0.5f * x[m][e] - 0.5f) + 0.25f;
#pragma unroll
      for (int v = 0; v < 3; ++v) y[m][v] = __builtin_fmaf(y[m][v], 0.5f, 0.75f);
    }
  }
  stamp(clk, 1);
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[m][i];
#pragma unroll
    for (int e = 0; e < (E > 0 ? E : 1); ++e) s += x[m][e];
#pragma unroll
    for (int v = 0; v < 3; ++v) s += y[m][v];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 256-byte rows, chunk c of row r stored at chunk c ^ (4 (r % 4) + (r / 4) % 4).
__device__ __forceinline__ int swz_off(int row, int byte) {
  const int c = byte >> 4;
  const int s = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * 256 + (((c ^ s) << 4) | (byte & 15));
}

// A 32 KiB tile of 128 rows. Per iteration a wavefront reads 16 KiB: mode 0
// as 16 ds_read_b128 (two 32-row blocks x 8 head-dim steps), mode 1 as 32
// ds_read_b64_tr_b16 (4 16-row steps x 4 column blocks x 2 row halves).
// Largest byte read: 16384 + 8192 + 31*256 + 255 (mode 0) and
// 16384 + 12288 + 15*256 + 255 (mode 1), both below 32768.
template <int MODE>
__global__ void __launch_bounds__(256) k_lds(unsigned* out, int iters, uint64_t* clk) {
  __shared__ __attribute__((aligned(16))) char tile[32768];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31, j = lane & 15;
  for (int i = tid; i < 32768 / 4; i += 256) ((unsigned*)tile)[i] = i * 2654435761u;
  __syncthreads();
  int off[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) off[kk] = swz_off(l32, (kk * 16 + 8 * g) * 2);
  int toff[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      toff[db][h] = swz_off(4 * g + 8 * h + (j >> 2), (db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)) * 2);
  u32x4 acc = {0u, 0u, 0u, 0u};
  stamp(clk, 0);
  for (int it = 0; it < iters; ++it) {
    const int base = (it & 1) * 16384;
    if constexpr (MODE == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc ^= *(const u32x4*)(tile + base + kb * 8192 + off[kk]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(tile + base + t * 4096 + toff[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(tile + base + t * 4096 + toff[db][1]));
          acc[db] ^= __builtin_bit_cast(u32x2, lo)[0] ^ __builtin_bit_cast(u32x2, hi)[1];
        }
    }
  }
  stamp(clk, 1);
  out[blockIdx.x * 256 + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// Launchers: `out` holds blocks x 256 elements (float, or unsigned for the
// LDS probe), `clk` 4 uint64 (device memory); 256 threads per block; the
// stream is a hipStream_t (null: the default stream). Return 0, or -1 on a
// bad argument or a launch error.
extern "C" int ml_mfma(float* out, int blocks, int iters, uint64_t* clk, void* stream) {
  if (!out || !clk || blocks <= 0 || iters <= 0) return -1;
  k_mfma<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, clk);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// with_mfma: 0 or 1; exps_per_mfma: 0 to 4.
extern "C" int ml_exp(float* out, int blocks, int iters, int with_mfma, int exps_per_mfma, uint64_t* clk,
                      void* stream) {
  if (!out || !clk || blocks <= 0 || iters <= 0) return -1;
  hipStream_t s = (hipStream_t)stream;
#define ML_EXP_CASE(E)                                                          \
  case E:                                                                       \
    if (with_mfma)                                                              \
      k_exp<true, E><<<blocks, 256, 0, s>>>(out, iters, clk);                   \
    else                                                                        \
      k_exp<false, E><<<blocks, 256, 0, s>>>(out, iters, clk);                  \
    break;
  switch (exps_per_mfma) {
    ML_EXP_CASE(0)
    ML_EXP_CASE(1)
    ML_EXP_CASE(2)
    ML_EXP_CASE(3)
    ML_EXP_CASE(4)
    default:
      return -1;
  }
#undef ML_EXP_CASE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// mode 0: ds_read_b128 rows; mode 1: ds_read_b64_tr_b16 transposes.
extern "C" int ml_lds(unsigned* out, int blocks, int iters, int mode, uint64_t* clk, void* stream) {
  if (!out || !clk || blocks <= 0 || iters <= 0 || (mode != 0 && mode != 1)) return -1;
  if (mode == 0)
    k_lds<0><<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, clk);
  else
    k_lds<1><<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, clk);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
