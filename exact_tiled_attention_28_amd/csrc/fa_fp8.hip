// fa_fp8.hip — FP8 (OCP e4m3) forward with incoherent processing for gfx950.
//
// The FlashAttention-3 news page ("Độ chính xác thấp FP8 và incoherent
// processing") quantizes Q and K to FP8 after multiplying both by the same
// random orthogonal matrix, a Hadamard transform with random signs: since
// (Q M)(K M)^T = Q K^T for orthogonal M, the scores are unchanged while
// large-magnitude outlier channels are spread over all channels, which
// lowers the quantization error; the transform costs O(d log d) per row.
//
// Two entry points:
//   * fa_quantize_fp8: y = FWHT(x o s) / sqrt(d) per row (s = +-1 signs; no
//     transform if none are given), then per 64-row block a power-of-two
//     scale 2^e, the smallest with max|y| <= 448 * 2^e, and e4m3 codes of
//     y / 2^e rounded to nearest, ties to even. Every step is exact or a
//     fixed sequence of fp32 operations (the butterflies a+b, a-b in stage
//     order h = 1, 2, ..., d/2, then one multiply by fp32(1/sqrt d)), so the
//     codes are reproducible bit for bit.
//   * fa_fwd_fp8: the forward of fa_fwd with S^T = K Q^T computed from the
//     codes by v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulate) and
//     scaled by the two block scales in fp32 before the softmax; P V stays in
//     bf16 as in fa_fwd.
#include <cfloat>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) int i32x8;

// ---------------------------------------------------------------------------
// e4m3 (OCP FP8 E4M3FN: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// largest finite 448, subnormal step 2^-9) codes of four values with
// |v| <= 448, round to nearest, ties to even, packed into one word (value j
// in byte j): gfx950's v_cvt_pk_fp8_f32 converts two fp32 values into two
// bytes of a word with exactly this rounding (checked bit for bit on
// [-448, 448] against the E4M3 definition, ties, subnormals, fp32 subnormals
// and signed zeros included).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned e4m3_word(float v0, float v1, float v2, float v3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  return (unsigned)w;
}

// The value of v in lane l ^ M (M = 1 or 2) of the same 4-lane quad: a DPP
// quad permutation, a plain vector move with no LDS round trip.
template <int M>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(M == 1 || M == 2, "within a quad");
  constexpr int kQuadPerm = M == 1 ? 0xB1 : 0x4E;  // lanes (1,0,3,2) or (2,3,0,1)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadPerm, 0xF, 0xF, false));
}

// Exponent e of the smallest power of two with amax <= 448 * 2^e (amax > 0,
// finite): with amax = m 2^E, m in [1, 2), and 448 = 1.75 2^8,
// e = E - 8 + (m > 1.75). Clamped to keep 2^e a normal fp32 number.
__device__ __forceinline__ int block_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const unsigned u = __float_as_uint(amax);
  const int E = (int)((u >> 23) & 0xFFu) - 127;
  const unsigned mant = u & 0x7FFFFFu;
  const int e = E - 8 + (mant > 0x600000u ? 1 : 0);  // m > 1.75 <=> mantissa bits > 0.75 * 2^23
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------------------
// Quantize pass: one workgroup (4 wavefronts) per 64-row block of one head.
// A row is spread over 4 lanes (a quad) holding D/4 consecutive elements
// each, so the butterflies of stages h < D/4 stay inside a lane and only the
// last two stages exchange values, with the lanes l ^ 1 and l ^ 2 of the same
// quad. A wavefront covers 16 rows, the workgroup the 64 rows of the block.
// (Measured at B8 H16 N2048 d128: 35 us per tensor, against 44 us with 16
// lanes per row and 52 us with one wavefront per block.)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) quantize_fp8_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales, const signed char* signs,
                                                            int N, int n_blocks) {
  constexpr int EPL = D / 4;  // elements per lane
  constexpr int NV = EPL / 8;  // 16-byte loads per lane
  __shared__ float wmax[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = blockIdx.x / n_blocks, blk = blockIdx.x % n_blocks;
  const int q = lane & 3;      // position in the quad
  const int c0 = q * EPL;      // first element of this lane
  const int row = blk * 64 + w * 16 + (lane >> 2);
  const size_t head_off = (size_t)head * N * D;

  float v[EPL];
  if (row < N) {
    const __bf16* xr = x + head_off + (size_t)row * D + c0;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const u32x4 raw = *(const u32x4*)(xr + 8 * u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * u + 2 * i] = __uint_as_float(raw[i] << 16);
        v[8 * u + 2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = 0.0f;
  }
  if (signs) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] *= (float)signs[c0 + e];
    // stages h = 1 .. EPL/2 inside the lane
#pragma unroll
    for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (!(e & h)) {
          const float a = v[e], b2 = v[e + h];
          v[e] = a + b2;
          v[e + h] = a - b2;
        }
    // stages h = EPL, 2 EPL across the quad: the partner holds element c +- h
#pragma unroll
    for (int m = 1; m <= 2; m <<= 1) {
      const bool lower = (q & m) == 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o = m == 1 ? quad_xor<1>(v[e]) : quad_xor<2>(v[e]);
        v[e] = lower ? v[e] + o : o - v[e];
      }
    }
    const float inv_sqrt_d = D == 64 ? 0.125f : 0.08838834764831845f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] *= inv_sqrt_d;
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(v[e]));
  // block max over the 4 wavefronts
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e2 = block_scale_exp(amax);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, e2);
  if (row < N) {
    uint8_t* cr = codes + head_off + (size_t)row * D + c0;
#pragma unroll
    for (int u = 0; u < EPL / 16; ++u) {
      u32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* t = v + 16 * u + 4 * i;
        out[i] = e4m3_word(ldexpf(t[0], -e2), ldexpf(t[1], -e2), ldexpf(t[2], -e2), ldexpf(t[3], -e2));
      }
      *(u32x4*)(cr + 16 * u) = out;
    }
  }
}

hipError_t launch_quantize_fp8(const void* x, void* codes, float* scales, const signed char* signs, int heads,
                               int N, int head_dim, hipStream_t s) {
  const int n_blocks = ceil_div(N, 64);
  const long long grid = (long long)heads * n_blocks;
  if (head_dim == 64)
    hipLaunchKernelGGL((quantize_fp8_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, (const __bf16*)x,
                       (uint8_t*)codes, scales, signs, N, n_blocks);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, (const __bf16*)x,
                       (uint8_t*)codes, scales, signs, N, n_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// V for the FP8 P V product: fa_quantize_vt_fp8 writes V transposed, one
// 64-key block at a time, as e4m3 codes of V / 2^e with the block's
// power-of-two scale 2^e (the same rule as above, no transform: only Q and K
// may be rotated). Layout [head][block][d][64]: row c of a block holds
// channel c of its 64 keys, in the order in which a lane of half-wave g of
// the FP8 product holds its probabilities: position 32 g + s, s < 32, holds
// key 32 (s / 16) + 8 ((s % 16) / 4) + 4 g + s % 4 of the block (the order of
// the S^T accumulator registers), so that the forward reads its A operand
// with plain 16-byte loads and feeds P from registers. Keys past the end get
// code 0. This is the transpose that the FP8 product needs, done once in the
// quantize pass that reads and rewrites V anyway.
// One workgroup per 64-key block of one head: the block goes through LDS
// (bf16, row-major), the block maximum by shuffles and 4 LDS words, and each
// thread writes whole 16-byte chunks of the transposed rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vt_key_of(int pos) {
  const int g = pos >> 5, s = pos & 31;
  return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * g + (s & 3);
}

template <int D>
__global__ void __launch_bounds__(256) quantize_vt_fp8_kernel(const __bf16* __restrict__ x,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales, int N, int n_blocks) {
  constexpr int RCH = D / 8;              // 16-byte chunks per bf16 row
  constexpr int LPT = 64 * RCH / 256;     // chunks loaded per thread
  constexpr int SPT = D * 4 / 256;        // 16-byte output chunks per thread
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * D];
  __shared__ float wmax[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = blockIdx.x / n_blocks, blk = blockIdx.x % n_blocks;
  const int k0 = blk * 64;
  const __bf16* xh = x + (size_t)head * N * D;

  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int ci = tid + 256 * u;
    const int row = ci / RCH, cc = ci % RCH;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (k0 + row < N) raw = *(const u32x4*)(xh + (size_t)(k0 + row) * D + 8 * cc);
    *(u32x4*)(tile + row * D + 8 * cc) = raw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[i] << 16)), fabsf(__uint_as_float(raw[i] & 0xFFFF0000u))));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e2 = block_scale_exp(amax);
  if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, e2);

  uint8_t* out = codes + (size_t)blockIdx.x * D * 64;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int oi = tid + 256 * u;
    const int c = oi >> 2, p0 = 16 * (oi & 3);  // channel c, positions p0 .. p0 + 15
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = ldexpf((float)tile[vt_key_of(p0 + 4 * i + j) * D + c], -e2);
      o[i] = e4m3_word(t[0], t[1], t[2], t[3]);
    }
    *(u32x4*)(out + c * 64 + p0) = o;
  }
}

hipError_t launch_quantize_vt_fp8(const void* v, void* codes, float* scales, int heads, int N, int head_dim,
                                  hipStream_t s) {
  const int n_blocks = ceil_div(N, 64);
  const long long grid = (long long)heads * n_blocks;
  if (head_dim == 64)
    hipLaunchKernelGGL((quantize_vt_fp8_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, (const __bf16*)v,
                       (uint8_t*)codes, scales, N, n_blocks);
  else
    hipLaunchKernelGGL((quantize_vt_fp8_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, (const __bf16*)v,
                       (uint8_t*)codes, scales, N, n_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 forward, d = 64 and 128: fwd_kernel's tiling (4 wavefronts x 32 query
// rows, 64-key tiles, K/V in LDS filled by HBM -> LDS loads) with the K tile
// held as e4m3 codes (d bytes per row: 8 KiB at d = 128, 4 KiB at 64) and
// S^T = K Q^T formed by d / 64 32x32x64 FP8 MFMAs per 32-key block. For those MFMAs a lane of
// half-wave g supplies, in both operands, the 32 codes of head-dim range
// [64 ks + 32 g, +32) of its key (A) or query (B) row: A and B then put the
// same channel in the same slot, and the output has the 32x32 layout of the
// bf16 MFMA. The 64-row scale blocks line up with the Q rows of a wavefront
// (32 rows inside one block) and with a K tile (64 rows = one block), so the
// scores of a tile are scaled by one scalar s_q s_k, folded into the base-2
// softmax constant.
// ---------------------------------------------------------------------------
// PV8: P V in FP8 as well (fa_fwd_fp8_pv): V arrives as the transposed codes
// of fa_quantize_vt_fp8 (tile j = 64 keys x D channels, contiguous, row c =
// channel c), P is packed to e4m3 at the fixed scale 2^8 straight from the
// S^T accumulator registers (whose order the V^T rows follow), and
// O^T += V^T P^T is one 32x32x64 FP8 product per 32 channels. The running
// sum l stays in fp32 over the unrounded probabilities; the V block scale of
// each tile is applied by keeping the accumulator in units of the current
// tile's scale (a power-of-two rescale, skipped while the scale repeats).
// QBF16: Q arrives in bf16 and is quantized here, exactly as
// fa_quantize_fp8 would (fa_fwd_fp8_quantize_q): each lane holds the head-dim
// ranges [64 ks + 32 g, +32) of its query row that its Q operand needs, the
// Hadamard butterflies run in the same stage order (h < 32 inside a range,
// h = 32 between the two half-waves, h = 64 between a lane's two ranges), the
// two wavefronts of a 64-row scale block exchange their maxima through LDS,
// and the codes go straight into the operand registers.
template <int D, bool CAUSAL, bool OUTF32, bool PV8 = false, bool QBF16 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_fp8_kernel(FwdArgs a) {
  constexpr int NW = 4, BR = 128, BC = 64, NKB = 2, NKS = D / 64, NDB = D / 32;
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  constexpr int KROWB = D, KRC = KROWB / 16, KTILEB = BC * KROWB, KCPW = KTILEB / (1024 * NW);  // fp8 K tile
  // V tile: bf16 rows of D channels, or (PV8) D rows of 64 key codes
  constexpr int VROWB = PV8 ? BC : D * 2, VRC = VROWB / 16, VTILEB = PV8 ? D * BC : BC * VROWB;
  constexpr int VCPW = VTILEB / (1024 * NW);
  static_assert(KTILEB % (1024 * NW) == 0 && VTILEB % (1024 * NW) == 0, "tiles must split into whole wave loads");

  // Three K buffers and two V buffers (56 KiB at d = 128): K_j is fetched two steps
  // before its scores, V_j one step before its product. Separate objects, so
  // that the compiler can tell the prefetch into one from reads of another.
  __shared__ __attribute__((aligned(16))) char sK0[KTILEB];
  __shared__ __attribute__((aligned(16))) char sV0[VTILEB];
  __shared__ __attribute__((aligned(16))) char sK1[KTILEB];
  __shared__ __attribute__((aligned(16))) char sV1[VTILEB];
  __shared__ __attribute__((aligned(16))) char sK2[KTILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const UnitItem ui = xcd_decode(blockIdx.x, a.B * a.Hkv);
  const int b = ui.unit / a.Hkv;
  const int hkv = ui.unit % a.Hkv;
  const int rank = ui.item / a.G;
  const int hq = hkv * a.G + ui.item % a.G;
  const int qt = CAUSAL ? (a.n_q_tiles - 1 - rank) : rank;
  const int q0 = qt * BR;
  const int q0w = q0 + 32 * w;
  const int qrow = q0w + l32;
  const int Nq = a.Nq, Nk = a.Nk;

  const size_t qhead = (size_t)(b * a.Hq + hq) * Nq;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * Nk;
  const char* __restrict__ Kh = uniform_ptr((const char*)a.k + kvhead * KROWB);
  // (PV8: the transposed code tiles of this K/V head, ceil(Nk / 64) tiles of
  // D * 64 bytes)
  const char* __restrict__ Vh =
      uniform_ptr((const char*)a.v + (PV8 ? (size_t)(b * a.Hkv + hkv) * ceil_div(Nk, 64) * (D * 64) : kvhead * VROWB));
  const int nqb = ceil_div(Nq, 64), nkb = ceil_div(Nk, 64);
  const float* __restrict__ sk = a.k_scales + (size_t)(b * a.Hkv + hkv) * nkb;

  // Q codes (B operand): 32 bytes of head-dim range [64 ks + 32 g, +32). A
  // negative scale flips the sign bit of every code (exact).
  i32x8 qf[NKS];
  float sq;
  if constexpr (QBF16) {
    __shared__ float qmax[NW];
    float v[NKS][32];
    {
      const __bf16* Qr = (const __bf16*)a.q + (qhead + qrow) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (qrow < Nq) x = *(const u32x4*)(Qr + 64 * ks + 32 * g + 8 * c);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[ks][8 * c + 2 * i] = __uint_as_float(x[i] << 16);
            v[ks][8 * c + 2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
          }
        }
    }
    if (a.q_signs) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 32; ++e) v[ks][e] *= (float)a.q_signs[64 * ks + 32 * g + e];
      // stages h = 1 .. 16 inside each 32-wide range
#pragma unroll
      for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int e = 0; e < 32; ++e)
            if (!(e & h)) {
              const float x0 = v[ks][e], x1 = v[ks][e + h];
              v[ks][e] = x0 + x1;
              v[ks][e + h] = x0 - x1;
            }
      // stage h = 32: element c of half-wave 0 with c + 32 of half-wave 1
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[ks][e]), __float_as_uint(v[ks][e]), false, false);
          const float o = __uint_as_float(g ? r[0] : r[1]);
          v[ks][e] = g ? o - v[ks][e] : v[ks][e] + o;
        }
      // stage h = 64 (d = 128): the lane's two ranges
      if constexpr (NKS == 2) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float x0 = v[0][e], x1 = v[1][e];
          v[0][e] = x0 + x1;
          v[1][e] = x0 - x1;
        }
      }
      const float inv_sqrt_d = D == 64 ? 0.125f : 0.08838834764831845f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 32; ++e) v[ks][e] *= inv_sqrt_d;
    }
    // maximum over the 64-row block: this wavefront's 32 rows and those of
    // wavefront w ^ 1 (rows past the end of Q are zeros, as in the pass)
    float amax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[ks][e]));
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    amax = half_swap_max(amax);
    if (lane == 0) qmax[w] = amax;
    __syncthreads();
    const int e2 = block_scale_exp(fmaxf(qmax[w], qmax[w ^ 1]));
    sq = ldexpf(1.0f, e2);
    const unsigned sign = a.neg ? 0x80808080u : 0u;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      unsigned wd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* t = v[ks] + 4 * i;
        wd[i] = e4m3_word(ldexpf(t[0], -e2), ldexpf(t[1], -e2), ldexpf(t[2], -e2), ldexpf(t[3], -e2)) ^ sign;
      }
      qf[ks] = i32x8{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3], (int)wd[4], (int)wd[5], (int)wd[6], (int)wd[7]};
    }
  } else {
    // A wavefront whose rows all lie past the end (last query tile) stores
    // nothing; its block index is clamped to stay inside the scale array.
    sq = a.q_scales[(size_t)(b * a.Hq + hq) * nqb + min(q0w >> 6, nqb - 1)];
    const char* Qr = (const char*)a.q + (qhead + qrow) * D;
    const unsigned sign = a.neg ? 0x80808080u : 0u;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
      if (qrow < Nq) {
        x0 = *(const u32x4*)(Qr + 64 * ks + 32 * g);
        x1 = *(const u32x4*)(Qr + 64 * ks + 32 * g + 16);
      }
      x0 ^= sign;
      x1 ^= sign;
      qf[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  }

  const int kv_end = kv_end_for(q0, BR, Nk, CAUSAL);
  const int n_kv = ceil_div(kv_end, BC);

  // HBM -> LDS staging of one K tile (codes) or one V tile (bf16): the
  // tile's scalar base plus this lane's 32-bit offset, computed once (kept
  // opaque so that the loads stay in the scalar-address form). In a tile that
  // runs past the end of K/V (FULL false), rows past the end read the last
  // row instead (their scores are masked).
  int kld[KCPW], vld[VCPW];
#pragma unroll
  for (int u = 0; u < KCPW; ++u) {
    const int idx = (wu * KCPW + u) * 64 + lane;
    const int row = idx / KRC;
    kld[u] = row * KROWB + (((idx % KRC) ^ swz<KRC>(row)) << 4);
  }
#pragma unroll
  for (int u = 0; u < VCPW; ++u) {
    const int idx = (wu * VCPW + u) * 64 + lane;
    const int row = idx / VRC;
    vld[u] = row * VROWB + (((idx % VRC) ^ swz<VRC>(row)) << 4);
  }
  auto issue = [&](auto full_tag, int jt, const char* __restrict__ Xh, const int* ld, auto ncpw, int rowb,
                   char* Xt) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int CPWX = decltype(ncpw)::value;
    const int kv0 = jt * BC;
    const char* Xb = uniform_ptr(Xh + (size_t)kv0 * (rowb != 0 ? rowb : D));
    const unsigned last = (unsigned)(Nk - 1 - kv0);  // last row of K/V in this tile
#pragma unroll
    for (int u = 0; u < CPWX; ++u) {
      unsigned ou = (unsigned)ld[u];
      if (!FULL && rowb != 0 && kv0 + BC > Nk && ou / rowb > last) ou = last * rowb + ou % rowb;
      asm volatile("" : "+v"(ou));
      load_lds_16(Xb, ou, Xt + (wu * CPWX + u) * 64 * 16);
    }
  };
  auto issue_k = [&](auto full_tag, int jt, char* Kt) __attribute__((always_inline)) {
    issue(full_tag, jt, Kh, kld, std::integral_constant<int, KCPW>{}, KROWB, Kt);
  };
  // (rowb 0: a transposed code tile, D bytes per key, never clamped)
  auto issue_v = [&](auto full_tag, int jt, char* Vt) __attribute__((always_inline)) {
    issue(full_tag, jt, Vh, vld, std::integral_constant<int, VCPW>{}, PV8 ? 0 : VROWB, Vt);
  };

  int koff[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) koff[ks][h] = tile_off<KRC>(l32, (4 * ks + 2 * g + h) * 16);
  int voff[NDB][2];
  if constexpr (PV8) {
    // A operand of the FP8 P V product: channel row 32 db + l32, the 32 codes
    // of half-wave g (two 16-byte reads); the swizzle of a 64-byte row depends
    // on the row mod 16 only, so channel blocks add constants
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[0][h] = tile_off<VRC>(l32, (2 * g + h) * 16);
  } else {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        voff[db][h] = tile_off<VRC>(4 * g + 8 * h + (j >> 2), (db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)) * 2);
  }
  // PV8: the V block scale the accumulator is currently expressed in
  const float* __restrict__ svp = PV8 ? a.v_scales + (size_t)(b * a.Hkv + hkv) * nkb : nullptr;
  float sv_ref = PV8 ? svp[0] : 1.0f;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;
  float lsum = 0.0f;
  // Last key this lane's query row may see (rows past the end of Q are
  // computed like the last row and not stored).
  const int last_key = CAUSAL ? min(qrow, Nk - 1) : Nk - 1;

  // c: |scale| log2(e) times the Q block scale and this tile's K block scale,
  // raised to at least the smallest normal float (a zero scale then gives
  // every visible key probability exactly 1 before normalisation)
  auto body = [&](auto mask_tag, int jt, const char* Kt, const char* Vt, float c, float sv) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kv0 = jt * BC;
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 k0 = *(const u32x4*)(Kt + koff[ks][0] + kb * 32 * KROWB);
        const u32x4 k1 = *(const u32x4*)(Kt + koff[ks][1] + kb * 32 * KROWB);
        const i32x8 ka = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3], (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf[ks], sacc[kb], 0, 0, 0, 0, 0, 0);
      }
    }
    // Key kv0 + kb*32 + 8*(r/4) + 4g + r%4 is visible iff it is at most
    // last_key: one compare of a constant with t per score. Masked scores
    // become -inf, which exp2 below turns into 0 (c is at least the smallest
    // normal float, so -inf * c stays -inf).
    if constexpr (MASK) {
      const int t = last_key - kv0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) <= t) ? sacc[kb][r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    const float mxs = half_swap_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mxs > m) != 0) {
      const float m_new = fmaxf(m, mxs);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    float rs = 0.0f;
    // PV8: P 2^8 (the FP8 codes' scale; l is kept scaled alike, exact)
    const float moff = PV8 ? 8.0f - m : -m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[kb][r], c, moff));
        sacc[kb][r] = p;
        rs += p;
      }
    lsum += rs;
    if constexpr (PV8) {
      // slot s = 16 kb + r of this half-wave: register r of block kb
      i32x8 pc;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = wd >> 2, r0 = 4 * (wd & 3);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][r0], sacc[kb][r0 + 1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][r0 + 2], sacc[kb][r0 + 3], x, true);
        pc[wd] = x;
      }
      if (sv != sv_ref) {  // uniform: a power-of-two change of units, exact
        const float f = sv_ref / sv;
        sv_ref = sv;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= f;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vb = Vt + db * 32 * VROWB;
        const u32x4 a0 = *(const u32x4*)(vb + voff[0][0]);
        const u32x4 a1 = *(const u32x4*)(vb + voff[0][1]);
        const i32x8 va = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pc, oacc[db], 0, 0, 0, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < BC / 16; ++t) {
      float pv[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) pv[v] = sacc[t >> 1][8 * (t & 1) + v];
      const bf16x8 pb = to_bf16x8(pv);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vp = Vt + 16 * t * VROWB;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(vp + voff[db][0]));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(vp + voff[db][1]));
        oacc[db] = mfma_bf16(cat4(lo, hi), pb, oacc[db]);
      }
    }
  };

  // Loads are issued in the order K_0, V_0, K_1 (here), then V_{j+1},
  // K_{j+2} at the top of step j, into K buffer j % 3 and V buffer j % 2.
  // Step j ends by waiting for K_{j+1} and V_{j+1} (loads retire in issue
  // order, so that is "at most the loads of K_{j+2} in flight"), then one
  // barrier, after all of the wavefront's LDS reads have completed, so the
  // loads of step j+1 may overwrite V_j and K_j. Steps before n_fast are
  // unmasked for every wavefront (Q tiles start at multiples of BR), and
  // both of their loads are whole tiles inside K/V; the others check
  // everything and take the masked body.
  constexpr int NTAIL = BR / BC;
  const int n_fast = max(0, min(min(n_kv - NTAIL, n_kv - 2), Nk / BC - 2));
  float c_next = 0.0f, c_cur = 0.0f;  // K block scale of the next tile; this tile's score factor
  float sv_next = 1.0f, sv_cur = sv_ref;  // PV8: V block scale of the next tile, of this tile
  auto step = [&](auto generic_tag, int jt, const char* Kt, const char* Vt, char* Vn, char* Kn2)
                  __attribute__((always_inline)) {
    constexpr bool GENERIC = decltype(generic_tag)::value;
    const bool has1 = !GENERIC || jt + 1 < n_kv;
    const bool has2 = !GENERIC || jt + 2 < n_kv;
    // The next tile's K block scale is loaded before this step's tile loads,
    // so the end-of-step wait covers it and nothing waits on it earlier.
    const float c = c_cur;
    const float sv = sv_cur;
    if (has1) c_next = sk[jt + 1];
    if constexpr (PV8)
      if (has1) sv_next = svp[jt + 1];
    if (has1) issue_v(std::bool_constant<!GENERIC>{}, jt + 1, Vn);
    if (has2) issue_k(std::bool_constant<!GENERIC>{}, jt + 2, Kn2);
    if constexpr (GENERIC) {
      if (!CAUSAL || jt * BC <= q0w + 31) body(std::true_type{}, jt, Kt, Vt, c, sv);
      if (has2)
        wait_vmem_n<KCPW>();
      else
        wait_vmem_n<0>();
    } else {
      body(std::false_type{}, jt, Kt, Vt, c, sv);
      wait_vmem_n<KCPW>();
    }
    c_cur = fmaxf(a.c * sq * c_next, FLT_MIN);
    sv_cur = sv_next;
    wait_lds();
    lds_barrier();
  };

  c_next = sk[0];
  issue_k(std::false_type{}, 0, sK0);
  issue_v(std::false_type{}, 0, sV0);
  if (n_kv > 1) {
    issue_k(std::false_type{}, 1, sK1);
    wait_vmem_n<KCPW>();
  } else {
    wait_vmem_n<0>();
  }
  __syncthreads();
  c_cur = fmaxf(a.c * sq * c_next, FLT_MIN);
  // Main loop unrolled over the six (K buffer, V buffer) phases, so that every
  // buffer is a compile-time choice; it can leave after any phase.
  int jt = 0;
  if (n_fast > 0) {
    while (true) {
      step(std::false_type{}, jt, sK0, sV0, sV1, sK2);
      if (++jt >= n_fast) break;
      step(std::false_type{}, jt, sK1, sV1, sV0, sK0);
      if (++jt >= n_fast) break;
      step(std::false_type{}, jt, sK2, sV0, sV1, sK1);
      if (++jt >= n_fast) break;
      step(std::false_type{}, jt, sK0, sV1, sV0, sK2);
      if (++jt >= n_fast) break;
      step(std::false_type{}, jt, sK1, sV0, sV1, sK0);
      if (++jt >= n_fast) break;
      step(std::false_type{}, jt, sK2, sV1, sV0, sK1);
      if (++jt >= n_fast) break;
    }
  }
  for (; jt < n_kv; ++jt) {
    switch (jt % 6) {
      case 0: step(std::true_type{}, jt, sK0, sV0, sV1, sK2); break;
      case 1: step(std::true_type{}, jt, sK1, sV1, sV0, sK0); break;
      case 2: step(std::true_type{}, jt, sK2, sV0, sV1, sK1); break;
      case 3: step(std::true_type{}, jt, sK0, sV1, sV0, sK2); break;
      case 4: step(std::true_type{}, jt, sK1, sV0, sV1, sK0); break;
      default: step(std::true_type{}, jt, sK2, sV1, sV0, sK1); break;
    }
  }

  const float lt = half_swap_add(lsum);
  // PV8: O = acc 2^e_v / (2^8 l), with lt = 2^8 l
  const float inv = (PV8 ? sv_ref : 1.0f) / lt;
  if (qrow < Nq) {
    const size_t orow = (qhead + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = db * 32 + 8 * a4 + 4 * g;
        f32x4 ov = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                    oacc[db][4 * a4 + 3] * inv};
        if constexpr (OUTF32)
          *(f32x4*)((float*)a.o + orow + d0) = ov;
        else
          *(bf16x4*)((__bf16*)a.o + orow + d0) = __builtin_convertvector(ov, bf16x4);
      }
    if (g == 0) a.lse[qhead + qrow] = (m + fast_log2(lt) - (PV8 ? 8.0f : 0.0f)) * kLn2;
  }
}

template <int D, bool PV8, bool QBF16>
static void launch_fwd_fp8_d(const FwdArgs& a, long long blocks, bool causal, bool out_f32, hipStream_t s) {
  if (causal) {
    if (out_f32)
      hipLaunchKernelGGL((fwd_fp8_kernel<D, true, true, PV8, QBF16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<D, true, false, PV8, QBF16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else {
    if (out_f32)
      hipLaunchKernelGGL((fwd_fp8_kernel<D, false, true, PV8, QBF16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<D, false, false, PV8, QBF16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
}

template <int D, bool QBF16>
static void launch_fwd_fp8_v(const FwdArgs& a, long long blocks, bool causal, bool out_f32, hipStream_t s) {
  if (a.v_scales != nullptr)
    launch_fwd_fp8_d<D, true, QBF16>(a, blocks, causal, out_f32, s);
  else
    launch_fwd_fp8_d<D, false, QBF16>(a, blocks, causal, out_f32, s);
}

hipError_t launch_fwd_fp8(const FwdArgs& a0, int head_dim, bool causal, bool out_f32, hipStream_t s) {
  FwdArgs a = a0;
  a.n_q_tiles = ceil_div(a.Nq, 128);
  const long long blocks = (long long)a.B * a.Hq * a.n_q_tiles;
  // q_scales null: Q is bf16 and quantized in the kernel
  const bool qbf16 = a.q_scales == nullptr;
  if (head_dim == 64) {
    if (qbf16)
      launch_fwd_fp8_v<64, true>(a, blocks, causal, out_f32, s);
    else
      launch_fwd_fp8_v<64, false>(a, blocks, causal, out_f32, s);
  } else {
    if (qbf16)
      launch_fwd_fp8_v<128, true>(a, blocks, causal, out_f32, s);
    else
      launch_fwd_fp8_v<128, false>(a, blocks, causal, out_f32, s);
  }
  return hipGetLastError();
}

}  // namespace fa
