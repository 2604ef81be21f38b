// fa_bwd.hip — exact attention backward for gfx950, FlashAttention-2 order.
//
// Method (page "6.2 FlashAttention V2 chi tiết", section 7; CSDN
// FlashAttention-2 article, "3.1.2 反向传播公式解析", "并行性 / 反向传播").
// fa_bwd (two passes, no atomics): bwd_dq_kernel (Q-outer) forms
// D = rowsum(dO o O) once per row (section 7.3), stores it, and sums dQ in
// registers; then bwd_dkdv_kernel (K/V-outer) forms dK and dV, reading D.
// fa_bwd_atomic (single pass, the scheme the pages describe first):
//   1. a separate preprocess kernel computes D = rowsum(dO o O) once and
//      zeroes the fp32 dQ accumulator (page 6.2, section 7.3);
//   2. the main kernel gives each workgroup one K/V column block j; it walks
//      every query head of the K/V head's group and every Q block i that can
//      see block j, recomputing P = exp(scale * Q_i K_j^T - L_i) from the
//      saved logsumexp (page 6.2, section 7.1), and accumulates
//        dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P o (dP - D_i),
//        dK_j += dS^T Q_i  (privately, in registers, so no atomics),
//        dQ_i += dS K_j    (added atomically to fp32 dQ in HBM, since many
//                           column blocks contribute to one Q block);
//      dQ and dK carry the factor `scale` of S = scale * Q K^T (chain rule).
//
// gfx950 mapping. The four wavefronts of a workgroup split the K/V block by
// keys (32 each), so dK and dV rows are private to one wavefront. Each
// wavefront computes S = Q_i K_j^T and dP = dO_i V_j^T as 32x32 blocks with
// one key per lane; K_j and V_j stay in registers as the B operands. The same
// accumulator layout is the B operand of dV^T += dO_i^T P and
// dK^T += Q_i^T dS, whose A operands are read from the LDS tiles of dO_i and
// Q_i with the gfx950 transpose read (ds_read_b64_tr_b16). dS is staged in
// LDS, transposed by key, and dQ_i = dS K_j is computed with both operands
// read by transpose reads, then added to HBM with fp32 atomics (lanes cover
// contiguous head-dim columns, so each atomic instruction touches whole
// cache lines).
#include <atomic>
#include <climits>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {

// ---------------------------------------------------------------------------
// preprocess: D = rowsum(dO o O), and dQ = 0 when dQ is accumulated atomically
// ---------------------------------------------------------------------------

template <int D, bool OF32, bool ZERO_DQ>
__global__ void __launch_bounds__(256) bwd_preprocess_kernel(const __bf16* __restrict__ dout, const void* __restrict__ o,
                                                             float* __restrict__ dvec, float* __restrict__ dq,
                                                             long long rows) {
  constexpr int LPR = D / 8;  // lanes per row: 8 elements each
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int part = (int)(t % LPR);
  float acc = 0.0f;
  if (row < rows) {
    const size_t base = (size_t)row * D + part * 8;
    const u32x4 dv = *(const u32x4*)(dout + base);
    const bf16x8 db = __builtin_bit_cast(bf16x8, dv);
    f32x8 of;
    if constexpr (OF32) {
      const f32x4 a = *(const f32x4*)((const float*)o + base);
      const f32x4 b = *(const f32x4*)((const float*)o + base + 4);
      of = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      const u32x4 ov = *(const u32x4*)((const __bf16*)o + base);
      of = __builtin_convertvector(__builtin_bit_cast(bf16x8, ov), f32x8);
    }
    const f32x8 df = __builtin_convertvector(db, f32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(df[e], of[e], acc);
    if constexpr (ZERO_DQ) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(dq + base) = z;
      *(f32x4*)(dq + base + 4) = z;
    }
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (row < rows && part == 0) dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// main backward kernel
// ---------------------------------------------------------------------------

template <int D>
struct BwdTile {
  static constexpr int NW = 4;
  static constexpr int BKV = 32 * NW;  // keys per workgroup (32 per wavefront)
  static constexpr int BQ = 64;        // query rows per step
  static constexpr int QROWB = D * 2;  // bytes per Q / dO / K row
  static constexpr int QRC = QROWB / 16;
  static constexpr int QTILEB = BQ * QROWB;
  static constexpr int KTILEB = BKV * QROWB;
  static constexpr int SROWB = BQ * 2;  // dS^T row: BQ bf16
  static constexpr int SRC = SROWB / 16;
  static constexpr int STILEB = BKV * SROWB;
  static constexpr int NT = 64 * NW;
  static constexpr int QCPW = QTILEB / (1024 * NW);  // HBM->LDS loads per wave per Q (or dO) tile
  static constexpr int KCPT = BKV * QRC / NT;
  static constexpr int NDB = D / 32;                 // 32-column blocks of the head dim
  static constexpr int NDQ = (BQ / 32) * NDB / NW;   // dQ 32x32 blocks per wave
  // LDS carve-up (bytes); the K tile and dS^T are only needed for atomic dQ
  static constexpr int OFF_Q = 0;                    // [2][QTILEB]
  static constexpr int OFF_DO = OFF_Q + 2 * QTILEB;  // [2][QTILEB]
  static constexpr int OFF_L = OFF_DO + 2 * QTILEB;  // [2][BQ] fp32 (L * log2 e)
  static constexpr int OFF_D = OFF_L + 2 * BQ * 4;   // [2][BQ] fp32
  static constexpr int OFF_K = OFF_D + 2 * BQ * 4;   // [KTILEB]
  static constexpr int OFF_S = OFF_K + KTILEB;       // [STILEB]
  static constexpr int LDS_BYTES_ATOMIC = OFF_S + STILEB;
  static constexpr int LDS_BYTES_SPLIT = OFF_K;
  static_assert(QTILEB % (1024 * NW) == 0 && BKV * QRC % NT == 0, "tiles must split evenly");
  static_assert((BQ / 32) * NDB % NW == 0 && NDQ >= 1, "dQ blocks must split evenly over waves");
};

// ATOMIC_DQ: also compute dQ_i += scale * dS K_j and add it to the fp32 dQ in
// HBM with atomics (the fused single-pass scheme). Without it the kernel
// produces dK and dV only and dQ comes from bwd_dq_kernel (second pass).
template <int D, bool CAUSAL, bool GF32, bool ATOMIC_DQ>
__global__ void __launch_bounds__(256) bwd_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int BKV = T::BKV, BQ = T::BQ, QROWB = T::QROWB, QRC = T::QRC, QTILEB = T::QTILEB, SRC = T::SRC;
  constexpr int NT = T::NT, QCPW = T::QCPW, KCPT = T::KCPT, NDQ = T::NDQ, NDB = T::NDB;
  constexpr int NKK = D / 16;  // K-steps of the S / dP products

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const sQ = smem + T::OFF_Q;
  char* const sDO = smem + T::OFF_DO;
  char* const sK = smem + T::OFF_K;
  char* const sS = smem + T::OFF_S;
  float* const sL = (float*)(smem + T::OFF_L);
  float* const sD = (float*)(smem + T::OFF_D);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same value, known to be wave-uniform
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int j16 = lane & 15;

  // Work decode: a unit is one (batch, K/V head), its items the K/V blocks
  // from the first (the heaviest under the causal mask) to the last;
  // units vary fastest (xcd_decode).
  const UnitItem ui = xcd_decode(blockIdx.x, a.B * a.Hkv);
  const int b = ui.unit / a.Hkv;
  const int hkv = ui.unit % a.Hkv;
  const int jblk = ui.item;
  const int kv0 = jblk * BKV;
  const int key_l = 32 * w + l32;  // this lane's key inside the block
  const int key = kv0 + key_l;

  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * a.Nk;
  const char* __restrict__ Kh = (const char*)a.k + kvhead * QROWB;
  const char* __restrict__ Vh = (const char*)a.v + kvhead * QROWB;

  // K_j, V_j rows of this lane's key as B operands (K^T and V^T columns).
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < a.Nk) {
      x = *(const u32x4*)(Kh + (size_t)key * QROWB + (kk * 16 + 8 * g) * 2);
      y = *(const u32x4*)(Vh + (size_t)key * QROWB + (kk * 16 + 8 * g) * 2);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, x);
    vf[kk] = __builtin_bit_cast(bf16x8, y);
  }
  // K_j tile in LDS for the dQ product.
  if constexpr (ATOMIC_DQ) {
#pragma unroll
    for (int u = 0; u < KCPT; ++u) {
      const int ci = tid + NT * u;
      const int row = ci / QRC, cc = ci % QRC;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kv0 + row < a.Nk) x = *(const u32x4*)(Kh + (size_t)(kv0 + row) * QROWB + cc * 16);
      *(u32x4*)(sK + tile_off<QRC>(row, cc * 16)) = x;
    }
  }

  // Per-lane LDS byte offsets, computed once. Row swizzles repeat every 8
  // rows, so whole 32-row blocks and 16-row steps only add constants.
  int qoff[NKK];  // A operand rows of Q / dO: row l32, head-dim step kk
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qoff[kk] = tile_off<QRC>(l32, (kk * 16 + 8 * g) * 2);
  int troff[NDB][2];  // transpose reads of Q / dO / K: column block db, half h
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      troff[db][h] = tile_off<QRC>(4 * g + 8 * h + (j16 >> 2), (db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2);
  int tsoff[BQ / 32][2];  // transpose reads of dS^T: query block qb, half h
#pragma unroll
  for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      tsoff[qb][h] = tile_off<SRC>(4 * g + 8 * h + (j16 >> 2), (qb * 32 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2);

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  const int n_qblk = ceil_div(a.Nq, BQ);
  const int i_first = first_q_tile_for(kv0, BQ, CAUSAL);
  const int n_i = n_qblk - i_first;
  const int total = a.G * n_i;
  const float c = a.c;
  const float scale = a.scale;

  // ---- Q_i / dO_i tiles: HBM -> swizzled LDS without registers; L_i, D_i
  // through registers (rows past the end get L = +inf, so P = 0 there) ----
  float lr = 0.0f, dr = 0.0f;
  auto issue_q = [&](int it, int buf) __attribute__((always_inline)) {
    const int hm = it / n_i;
    const int i = i_first + it % n_i;
    const int hq = hkv * a.G + hm;
    const size_t qhead = (size_t)(b * a.Hq + hq) * a.Nq;
    const int q0 = i * BQ;
    const char* Qb = uniform_ptr((const char*)a.q + (qhead + q0) * QROWB);
    const char* Ob = uniform_ptr((const char*)a.dout + (qhead + q0) * QROWB);
#pragma unroll
    for (int u = 0; u < QCPW; ++u) {
      const int cb = (wu * QCPW + u) * 64;
      const int idx = cb + lane;
      const int row = idx / QRC, pc = idx % QRC;
      const int lc = pc ^ swz<QRC>(row);
      const unsigned off = (unsigned)(min(row, a.Nq - 1 - q0) * QROWB + lc * 16);
      load_lds_16(Qb, off, sQ + buf * QTILEB + cb * 16);
      load_lds_16(Ob, off, sDO + buf * QTILEB + cb * 16);
    }
    if (tid < BQ) {
      const bool ok = q0 + tid < a.Nq;
      lr = ok ? a.lse[qhead + q0 + tid] * kLog2e : INFINITY;
      dr = ok ? a.dvec[qhead + q0 + tid] : 0.0f;
    }
  };
  auto store_ld = [&](int buf) __attribute__((always_inline)) {
    if (tid < BQ) {
      sL[buf * BQ + tid] = lr;
      sD[buf * BQ + tid] = dr;
    }
  };

  if (total > 0) {
    issue_q(0, 0);
    store_ld(0);
  }
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    const int hm = it / n_i;
    const int i = i_first + it % n_i;
    const int hq = hkv * a.G + hm;
    const size_t qhead = (size_t)(b * a.Hq + hq) * a.Nq;
    const int q0 = i * BQ;
    const bool has_next = it + 1 < total;
    if (has_next) issue_q(it + 1, buf ^ 1);

    const char* tQ = sQ + buf * QTILEB;
    const char* tDO = sDO + buf * QTILEB;
    const float* tL = sL + buf * BQ;
    const float* tD = sD + buf * BQ;

    // A wavefront whose keys all lie after every query of this block skips
    // the products; its dS^T rows are written as zeros.
    const bool active = !CAUSAL || kv0 + 32 * w <= q0 + BQ - 1;
    bf16x8 dsb[BQ / 16];
    if (active) {
      // ---- S = Q_i K_j^T (one key per lane, query rows in registers) -------
      f32x16 s[BQ / 32];
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        s[qb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          s[qb] = mfma_bf16(*(const bf16x8*)(tQ + qoff[kk] + qb * 32 * QROWB), kf[kk], s[qb]);
      }
      // ---- P = exp2(S c - L log2 e) --------------------------------------------
      const bool need_mask = (CAUSAL && kv0 + 32 * w + 31 > q0) || (kv0 + 32 * w + 32 > a.Nk);
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int r0 = qb * 32 + 8 * a4 + 4 * g;
          const f32x4 lv = *(const f32x4*)(tL + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p = fast_exp2(fmaf(s[qb][4 * a4 + e], c, -lv[e]));
            if (need_mask) {
              const bool vis = key < a.Nk && (!CAUSAL || key <= q0 + r0 + e);
              p = vis ? p : 0.0f;
            }
            s[qb][4 * a4 + e] = p;
          }
        }
      // ---- dV^T += dO_i^T P ------------------------------------------------------
#pragma unroll
      for (int t = 0; t < BQ / 16; ++t) {
        float pv[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) pv[v] = s[t >> 1][8 * (t & 1) + v];
        const bf16x8 pb = to_bf16x8(pv);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* base = tDO + 16 * t * QROWB;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[db][1]));
          dvacc[db] = mfma_bf16(cat4(lo, hi), pb, dvacc[db]);
        }
      }
      // ---- dP = dO_i V_j^T, dS = P o (dP - D) -----------------------------------
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        f32x16 dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          dp = mfma_bf16(*(const bf16x8*)(tDO + qoff[kk] + qb * 32 * QROWB), vf[kk], dp);
        float dsv[16];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 dv = *(const f32x4*)(tD + qb * 32 + 8 * a4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) dsv[4 * a4 + e] = s[qb][4 * a4 + e] * (dp[4 * a4 + e] - dv[e]);
        }
        dsb[2 * qb] = to_bf16x8(dsv);
        dsb[2 * qb + 1] = to_bf16x8(dsv + 8);
      }
      // ---- dK^T += Q_i^T dS --------------------------------------------------------
#pragma unroll
      for (int t = 0; t < BQ / 16; ++t)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* base = tQ + 16 * t * QROWB;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[db][1]));
          dkacc[db] = mfma_bf16(cat4(lo, hi), dsb[t], dkacc[db]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < BQ / 16; ++t) dsb[t] = bf16x8{};
    }

    if constexpr (ATOMIC_DQ) {
      // ---- stage dS^T (keys x queries, bf16): register 4*a4+e of block qb
      // holds query qb*32 + 8*a4 + 4g + e -----------------------------------------
#pragma unroll
      for (int t = 0; t < BQ / 16; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int col = (t >> 1) * 32 + 8 * (2 * (t & 1) + hh) + 4 * g;
          const bf16x4 v4 = {dsb[t][4 * hh], dsb[t][4 * hh + 1], dsb[t][4 * hh + 2], dsb[t][4 * hh + 3]};
          *(bf16x4*)(sS + tile_off<SRC>(key_l, col * 2)) = v4;
        }
      __syncthreads();

      // ---- dQ_i += scale * dS K_j (fp32 atomics) --------------------------------
#pragma unroll
      for (int u = 0; u < NDQ; ++u) {
        const int bi = w + T::NW * u;
        const int qb = bi / NDB, db = bi % NDB;
        if (!CAUSAL || q0 + qb * 32 + 31 >= kv0) {
          f32x16 acc = f32x16{};
#pragma unroll
          for (int t = 0; t < BKV / 16; ++t) {
            const char* sb = sS + 16 * t * T::SROWB;
            const char* kb = sK + 16 * t * QROWB;
            const short4v slo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(sb + tsoff[qb][0]));
            const short4v shi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(sb + tsoff[qb][1]));
            const short4v klo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(kb + troff[db][0]));
            const short4v khi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(kb + troff[db][1]));
            acc = mfma_bf16(cat4(slo, shi), cat4(klo, khi), acc);
          }
          float* dqh = a.dq + qhead * D;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qrow = q0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (qrow < a.Nq) atomicAdd(dqh + (size_t)qrow * D + db * 32 + l32, scale * acc[r]);
          }
        }
      }
    }

    if (has_next) store_ld(buf ^ 1);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T, one key per lane ------------
  if (key < a.Nk) {
    const size_t rowoff = (kvhead + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = db * 32 + 8 * a4 + 4 * g;
        const f32x4 kv = {scale * dkacc[db][4 * a4], scale * dkacc[db][4 * a4 + 1], scale * dkacc[db][4 * a4 + 2],
                          scale * dkacc[db][4 * a4 + 3]};
        const f32x4 vv = {dvacc[db][4 * a4], dvacc[db][4 * a4 + 1], dvacc[db][4 * a4 + 2], dvacc[db][4 * a4 + 3]};
        if constexpr (GF32) {
          *(f32x4*)((float*)a.dk + rowoff + d0) = kv;
          *(f32x4*)((float*)a.dv + rowoff + d0) = vv;
        } else {
          *(bf16x4*)((__bf16*)a.dk + rowoff + d0) = __builtin_convertvector(kv, bf16x4);
          *(bf16x4*)((__bf16*)a.dv + rowoff + d0) = __builtin_convertvector(vv, bf16x4);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV pass of the two-pass scheme: 8 wavefronts, 2 per SIMD
// ---------------------------------------------------------------------------
//
// Same method as bwd_kernel without dQ. The workgroup owns a K/V column block
// of 128 keys and walks every Q block of 64 rows (of every query head of the
// group) that can see it. Wavefront w = (kg, h), kg = w mod 4, h = w / 4,
// owns the 32 keys 32*kg.. of the block: their K and V rows stay in its
// registers for the whole loop as the B operands of S = Q K^T and
// dP = dO V^T, which it forms for the 32 query rows 32*h.. of each Q block.
// Its dK, dV accumulators cover only head-dim half h (32 keys x D/2 each).
// The two wavefronts with the same keys swap their P and dS (bf16, exactly
// the registers that feed the products) through LDS once per Q block, so each
// adds all 64 query rows to its half of dV^T += dO^T P and dK^T += Q^T dS.
// Compared with each wavefront accumulating the full head dimension for its
// own 32 query rows and summing the halves at the end, this halves the
// accumulator registers, which pays for K and V in registers (no K/V operand
// reads from LDS) and leaves room for the scheduler.
template <int D, bool HILO = false>
struct DkdvTile {
  static constexpr int NW = 8;
  static constexpr int BKV = 128, BQ = 64;
  static constexpr int ROWB = D * 2, RC = ROWB / 16;
  static constexpr int QTILEB = BQ * ROWB;
  static constexpr int QCPW = QTILEB / (1024 * NW);
  // per wavefront: P and dS, 2 x bf16x8 each per lane (and their low halves
  // when they are carried as bf16 pairs)
  static constexpr int XB = (HILO ? 8 : 4) * 64 * 16;
  // LDS (static): exchange [NW][XB], Q and dO tiles x 2, L and D x 2
  static constexpr int LDS_BYTES = NW * XB + 4 * QTILEB + 4 * BQ * 4;
  static_assert(QTILEB % (1024 * NW) == 0, "tiles must split evenly");
  static_assert(D % 64 == 0, "each wavefront takes whole 32-wide head-dim blocks of one half");
};

// HILO: P and dS enter the dV and dK products as bf16 pairs hi + lo (two
// products each, see bf16_residual8) instead of one bf16 rounding.
template <int D, bool CAUSAL, bool GF32, bool VARLEN = false, bool HILO = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dkdv_kernel(BwdArgs a) {
  using T = DkdvTile<D, HILO>;
  constexpr int BKV = T::BKV, BQ = T::BQ, ROWB = T::ROWB, RC = T::RC, QTILEB = T::QTILEB;
  // Own query half's dV/dK products before the exchange barrier: +2.5-5 % on
  // causal d = 128 backward shapes on MI355X and +1.5-3 % non-causal; HILO
  // keeps them after it (it reads its own P and dS back from the exchange).
  constexpr bool OWN_FIRST = !HILO;
  constexpr int QCPW = T::QCPW, XB = T::XB;
  constexpr int NKK = D / 16, NDH = D / 64;  // NDH: 32-wide head-dim blocks per half

  // Static LDS, one object per buffer: with the loop unrolled over the two
  // Q/dO buffers every LDS access names its buffer at compile time, so the
  // compiler can tell that the reads of one buffer never alias the HBM->LDS
  // loads in flight into the other and does not wait for them.
  // Each buffer holds its Q tile and then its dO tile. The compiler lays the
  // static LDS objects out by decreasing alignment, so the two buffers come
  // first (at 0 and 32 KiB) and every tile address is a loop-invariant
  // per-lane offset plus a constant that fits the 16-bit immediate offset of
  // the LDS reads: no address arithmetic per read (-30 VALU instructions per
  // Q block, +3-4 % on causal d = 128 backward shapes).
  __shared__ __attribute__((aligned(1024))) char sQD0[2 * QTILEB];
  __shared__ __attribute__((aligned(1024))) char sQD1[2 * QTILEB];
  __shared__ __attribute__((aligned(16))) char sX[T::NW * XB];
  char* const sQ0 = sQD0;
  char* const sDO0 = sQD0 + QTILEB;
  char* const sQ1 = sQD1;
  char* const sDO1 = sQD1 + QTILEB;
  __shared__ __attribute__((aligned(16))) float sL0[BQ];
  __shared__ __attribute__((aligned(16))) float sL1[BQ];
  __shared__ __attribute__((aligned(16))) float sD0[BQ];
  __shared__ __attribute__((aligned(16))) float sD1[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same value, known to be wave-uniform
  const int kg = w & 3;  // key group: keys 32*kg.. of the block
  const int h = w >> 2;  // query half for S and dP, head-dim half for dK and dV
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int j16 = lane & 15;

  const UnitItem ui = xcd_decode(blockIdx.x, a.B * a.Hkv);
  const int b = ui.unit / a.Hkv;
  const int hkv = ui.unit % a.Hkv;
  const int kv0 = ui.item * BKV;
  const int key = kv0 + 32 * kg + l32;  // this lane's key

  // Sequence lengths and head bases: fixed-length [B][H][N][d], or a packed
  // variable-length batch [H][total][d] (a.Nq / a.Nk are then the longest
  // lengths); q_base(hq) is the first row of query head hq of this sequence.
  int Nq = a.Nq, Nk = a.Nk;
  size_t kvhead;
  int q_off = 0;
  if constexpr (VARLEN) {
    const SeqSpan sq = clamp_span(a.cu_q[b], a.cu_q[b + 1], a.total_q, a.Nq);
    const SeqSpan sk = clamp_span(a.cu_k[b], a.cu_k[b + 1], a.total_k, a.Nk);
    Nq = sq.len;
    Nk = sk.len;
    if (kv0 >= Nk) return;  // the whole key block lies past this sequence
    q_off = sq.off;
    kvhead = (size_t)hkv * a.total_k + sk.off;
  } else {
    kvhead = (size_t)(b * a.Hkv + hkv) * a.Nk;
  }
  auto q_base = [&](int hq) __attribute__((always_inline)) -> size_t {
    if constexpr (VARLEN) return (size_t)hq * a.total_q + q_off;
    return (size_t)(b * a.Hq + hq) * a.Nq;
  };

  // K and V rows of this lane's key as B operands: head-dim elements
  // 16*kk + 8*g .. +7 (zero past the end of K/V).
  bf16x8 kf[NKK], vf[NKK];
  {
    const bool ok = key < Nk;
    const size_t row = (kvhead + (ok ? key : 0)) * ROWB;
    const char* Kr = (const char*)a.k + row;
    const char* Vr = (const char*)a.v + row;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (ok) {
        x = *(const u32x4*)(Kr + (kk * 16 + 8 * g) * 2);
        y = *(const u32x4*)(Vr + (kk * 16 + 8 * g) * 2);
      }
      kf[kk] = __builtin_bit_cast(bf16x8, x);
      vf[kk] = __builtin_bit_cast(bf16x8, y);
    }
  }

  // Per-lane LDS offsets.
  // row reads: row 32*h + l32 of a Q block, head-dim step kk (the swizzle
  // depends on the row mod 16, so the half's offset is part of it)
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = tile_off<RC>(32 * h + l32, (kk * 16 + 8 * g) * 2);
  // transpose reads: this wavefront's head-dim blocks db, rows +8*e of the
  // query half of its own scores (ptr = 0) or of its partner's (ptr = 1)
  int troff[2][NDH][2];
#pragma unroll
  for (int ptr = 0; ptr < 2; ++ptr)
#pragma unroll
    for (int db = 0; db < NDH; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        troff[ptr][db][e] = tile_off<RC>(32 * (h ^ ptr) + 4 * g + 8 * e + (j16 >> 2),
                                         ((h * NDH + db) * 32 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2);

  f32x16 dkacc[NDH], dvacc[NDH];
#pragma unroll
  for (int db = 0; db < NDH; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  const int n_qblk = ceil_div(Nq, BQ);
  const int i_first = first_q_tile_for(kv0, BQ, CAUSAL);
  const int n_i = n_qblk - i_first;
  const int total = a.G * n_i;
  const float c = a.c;
  const float scale = a.scale;

  // The next Q block's L and D are loaded into registers as its Q/dO tiles
  // are issued and only used (scaled, masked, stored to LDS) at the end of
  // the current block: using them at once would make the wavefront wait for
  // every load in flight, the tiles just issued included.
  float lr = 0.0f, dr = 0.0f;
  bool lok = false;
  auto issue_q = [&](int it, char* nQ, char* nDO) __attribute__((always_inline)) {
    const int hm = it / n_i;
    const int i = i_first + it % n_i;
    const int hq = hkv * a.G + hm;
    const size_t qhead = q_base(hq);
    const int q0 = i * BQ;
    if (tid < BQ) {
      lok = q0 + tid < Nq;
      const size_t r = qhead + q0 + (lok ? tid : 0);  // row q0 < Nq exists
      lr = a.lse[r];
      dr = a.dvec[r];
    }
    // Scalar tile base plus a 32-bit per-lane offset (rows past the end of
    // Q read the last row); both are kept opaque so that the loads stay in
    // the scalar-address form.
    const char* Qb = uniform_ptr((const char*)a.q + (qhead + q0) * ROWB);
    const char* Ob = uniform_ptr((const char*)a.dout + (qhead + q0) * ROWB);
    const int last = Nq - 1 - q0;
#pragma unroll
    for (int u = 0; u < QCPW; ++u) {
      const int cb = (wu * QCPW + u) * 64;
      const int idx = cb + lane;
      const int row = idx / RC, pc = idx % RC;
      const int lc = pc ^ swz<RC>(row);
      unsigned off = (unsigned)(min(row, last) * ROWB + lc * 16);
      asm volatile("" : "+v"(off));
      load_lds_16(Qb, off, nQ + cb * 16);
      load_lds_16(Ob, off, nDO + cb * 16);
    }
  };
  auto store_ld = [&](float* nL, float* nD) __attribute__((always_inline)) {
    if (tid < BQ) {
      nL[tid] = lok ? lr * kLog2e : INFINITY;
      nD[tid] = lok ? dr : 0.0f;
    }
  };

  if (total > 0) {
    issue_q(0, sQ0, sDO0);
    store_ld(sL0, sD0);
  }
  wait_vmem();
  __syncthreads();

  char* const myX = sX + w * XB;
  const char* const ptX = sX + (w ^ 4) * XB;

  // P and dS of this wavefront's 32 x 32 block (keys x its query half).
  // With HILO, pl and dsl receive the low halves of P and dS.
  auto scores = [&](auto mask_tag, int q0, const char* tQ, const char* tDO, const float* tL, const float* tD,
                    bf16x8 (&pb)[2], bf16x8 (&dsb)[2], bf16x8 (&pl)[2], bf16x8 (&dsl)[2])
                    __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* qRows = tQ;
    const char* oRows = tDO;
    // S = Q K^T (query rows from LDS, K rows in registers, one key per lane)
    f32x16 s = f32x16{};
    {
      // The Q operand of step kk + 1 is read before the product of step kk,
      // order pinned (measured 1-2 % faster).
      bf16x8 qa[2];
      qa[0] = *(const bf16x8*)(qRows + roff[0]);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) qa[(kk + 1) & 1] = *(const bf16x8*)(qRows + roff[kk + 1]);
        s = mfma_bf16(qa[kk & 1], kf[kk], s);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 2 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    // P = exp2(S c - L log2 e). Masked: query q0 + 32h + 8*a4 + 4g + e sees
    // this lane's key iff 8*a4 + e >= tq (no query if the key is past the end
    // of K, every query without the causal mask).
    const int tq = key >= Nk ? INT_MAX : (CAUSAL ? key - q0 - 32 * h - 4 * g : INT_MIN);
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int r0 = h * 32 + 8 * a4 + 4 * g;
      const f32x4 lv = *(const f32x4*)(tL + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = fast_exp2(fmaf(s[4 * a4 + e], c, -lv[e]));
        if constexpr (MASK) p = (8 * a4 + e >= tq) ? p : 0.0f;
        s[4 * a4 + e] = p;
      }
    }
    {
      float pv[8];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int v = 0; v < 8; ++v) pv[v] = s[8 * t + v];
        pb[t] = to_bf16x8(pv);
        if constexpr (HILO) pl[t] = bf16_residual8(pv, pb[t]);
      }
    }
    // dP = dO V^T, dS = P o (dP - D)
    f32x16 dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) dp = mfma_bf16(*(const bf16x8*)(oRows + roff[kk]), vf[kk], dp);
    float dsv[16];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x4 dv = *(const f32x4*)(tD + h * 32 + 8 * a4 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dsv[4 * a4 + e] = s[4 * a4 + e] * (dp[4 * a4 + e] - dv[e]);
    }
    dsb[0] = to_bf16x8(dsv);
    dsb[1] = to_bf16x8(dsv + 8);
    if constexpr (HILO) {
      dsl[0] = bf16_residual8(dsv, dsb[0]);
      dsl[1] = bf16_residual8(dsv + 8, dsb[1]);
    }
  };

  // dV^T += dO^T P and dK^T += Q^T dS over the 32 query rows of the
  // wavefront's own query half (ptr = 0) or its partner's (ptr = 1), for this
  // wavefront's head-dim half (with HILO, also the products of the low halves
  // pl, dsl; unused otherwise).
  auto grads = [&](int ptr, const char* tQ, const char* tDO, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2],
                   const bf16x8 (&pl)[2], const bf16x8 (&dsl)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
        const char* base = tDO + 16 * t * ROWB;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[ptr][db][0]));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[ptr][db][1]));
        dvacc[db] = mfma_bf16(cat4(lo, hi), pb[t], dvacc[db]);
        if constexpr (HILO) dvacc[db] = mfma_bf16(cat4(lo, hi), pl[t], dvacc[db]);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
        const char* base = tQ + 16 * t * ROWB;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[ptr][db][0]));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(base + troff[ptr][db][1]));
        dkacc[db] = mfma_bf16(cat4(lo, hi), dsb[t], dkacc[db]);
        if constexpr (HILO) dkacc[db] = mfma_bf16(cat4(lo, hi), dsl[t], dkacc[db]);
      }
  };
  // The four (or eight, with HILO) bf16x8 exchange slots of a wavefront:
  // P hi, dS hi, then P lo, dS lo.
  auto read_x = [&](const char* X, bf16x8 (&pb)[2], bf16x8 (&dsb)[2], bf16x8 (&pl)[2], bf16x8 (&dsl)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pb[t] = *(const bf16x8*)(X + (t * 64 + lane) * 16);
      dsb[t] = *(const bf16x8*)(X + ((2 + t) * 64 + lane) * 16);
      if constexpr (HILO) {
        pl[t] = *(const bf16x8*)(X + ((4 + t) * 64 + lane) * 16);
        dsl[t] = *(const bf16x8*)(X + ((6 + t) * 64 + lane) * 16);
      }
    }
  };

  // One Q block: its tiles in (tQ, tDO, tL, tD), the next block's loads go to
  // (nQ, nDO, nL, nD).
  auto block = [&](int it, const char* tQ, const char* tDO, const float* tL, const float* tD, char* nQ, char* nDO,
                   float* nL, float* nD) __attribute__((always_inline)) {
    const int i = i_first + it % n_i;
    const int q0 = i * BQ;
    const bool has_next = it + 1 < total;
    if (has_next) issue_q(it + 1, nQ, nDO);
    // A (key group, query half) block is skipped when all its keys lie after
    // all its queries.
    const bool act0 = !CAUSAL || kv0 + 32 * kg <= q0 + 31;
    const bool act1 = !CAUSAL || kv0 + 32 * kg <= q0 + 63;
    const bool mine = h ? act1 : act0;
    bf16x8 pb[2] = {}, dsb[2] = {}, pl[2] = {}, dsl[2] = {};
    if (mine) {
      const bool need_mask = (CAUSAL && kv0 + 32 * kg + 31 > q0 + 32 * h) || (kv0 + 32 * kg + 32 > Nk);
      if (need_mask)
        scores(std::true_type{}, q0, tQ, tDO, tL, tD, pb, dsb, pl, dsl);
      else
        scores(std::false_type{}, q0, tQ, tDO, tL, tD, pb, dsb, pl, dsl);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        *(bf16x8*)(myX + (t * 64 + lane) * 16) = pb[t];
        *(bf16x8*)(myX + ((2 + t) * 64 + lane) * 16) = dsb[t];
        if constexpr (HILO) {
          *(bf16x8*)(myX + ((4 + t) * 64 + lane) * 16) = pl[t];
          *(bf16x8*)(myX + ((6 + t) * 64 + lane) * 16) = dsl[t];
        }
      }
      // The products of the wavefront's own query half need nothing from
      // its partner: with OWN_FIRST they run before the exchange barrier,
      // which then waits only for what is left of the partner's scores.
      if constexpr (OWN_FIRST) grads(0, tQ, tDO, pb, dsb, pl, dsl);
    }
    // The exchange needs only the P/dS writes to have landed; the Q/dO tiles
    // of the next block stay in flight across this barrier.
    wait_lds();
    lds_barrier();
    if (!OWN_FIRST && mine) {
      // With HILO the wavefront's own P and dS are read back from the
      // exchange rather than kept in registers across the barrier.
      if constexpr (HILO) read_x(myX, pb, dsb, pl, dsl);
      grads(0, tQ, tDO, pb, dsb, pl, dsl);
    }
    if (h ? act0 : act1) {
      bf16x8 ppb[2], pds[2], ppl[2], pdsl[2];
      read_x(ptX, ppb, pds, ppl, pdsl);
      grads(1, tQ, tDO, ppb, pds, ppl, pdsl);
    }
    if (has_next) store_ld(nL, nD);
    wait_vmem();
    __syncthreads();
  };
  for (int it = 0; it < total; it += 2) {
    block(it, sQ0, sDO0, sL0, sD0, sQ1, sDO1, sL1, sD1);
    if (it + 1 >= total) break;
    block(it + 1, sQ1, sDO1, sL1, sD1, sQ0, sDO0, sL0, sD0);
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T for this head-dim half --------
  if (key < Nk) {
    const size_t rowoff = (kvhead + key) * D;
#pragma unroll
    for (int db = 0; db < NDH; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = (h * NDH + db) * 32 + 8 * a4 + 4 * g;
        const f32x4 kv = {scale * dkacc[db][4 * a4], scale * dkacc[db][4 * a4 + 1], scale * dkacc[db][4 * a4 + 2],
                          scale * dkacc[db][4 * a4 + 3]};
        const f32x4 vv = {dvacc[db][4 * a4], dvacc[db][4 * a4 + 1], dvacc[db][4 * a4 + 2], dvacc[db][4 * a4 + 3]};
        if constexpr (GF32) {
          *(f32x4*)((float*)a.dk + rowoff + d0) = kv;
          *(f32x4*)((float*)a.dv + rowoff + d0) = vv;
        } else {
          *(bf16x4*)((__bf16*)a.dk + rowoff + d0) = __builtin_convertvector(kv, bf16x4);
          *(bf16x4*)((__bf16*)a.dv + rowoff + d0) = __builtin_convertvector(vv, bf16x4);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dK/dV pass with four independent wavefronts: bwd_dkdv4_kernel
// ---------------------------------------------------------------------------
//
// The same K/V-outer loop (page 6.2, section 7.2) with a layout that needs no
// exchange between wavefronts: a workgroup owns a 64-key block and each of its
// four wavefronts owns 16 of those keys outright. With the 16x16x32 bf16
// MFMA a wavefront forms S = Q K^T and dP = dO V^T for all 64 query rows of a
// Q block against its 16 keys (one key per lane column, K and V rows in
// registers as B operands), and accumulates dV^T += dO^T P and dK^T += Q^T dS
// over the full head dimension (16 keys x D, 2 x D/16 fp32 per lane). The
// only workgroup barrier per Q block protects the double-buffered Q/dO/L/D
// tiles (4 x 64 rows + L/D: 33 KiB at d = 64), so several workgroups share a
// CU and their wavefronts interleave matrix and vector work on each SIMD
// independently. The 16x16 products read twice the operand bytes per flop of
// the 32x32 ones, so the kernel serves d = 64, where it is the faster layout.
//
// 16x16x32 MFMA layouts (gfx950): A (16 x 32): lane l holds row l % 16 and 8
// k values chosen by the lane group G = l / 16; B (32 x 16): column l % 16,
// the same k set; C (16 x 16, 4 fp32): column l % 16, rows 4G + i. S comes out
// with lane l holding key l % 16 for queries 16 mb + 4G + i (m-block mb); two
// m-blocks (2t, 2t + 1) form the 8 k slots of the products' B operand, and the
// A operands (dO^T, Q^T) are transpose reads of exactly those query rows.
//
// LDS rows use the swizzle dkdv4_swz, which keeps both operand reads free of
// bank conflicts: ds_read_b128 of 16 consecutive rows at one chunk (a
// bijection on row % 16), and ds_read_b64_tr_b16 of rows 8h .. 8h + 7 over an
// aligned pair of chunks (the 8 rows move the pair to 8 different pairs).
template <int ROW_CHUNKS>
__device__ __forceinline__ int dkdv4_swz(int row) {
  if constexpr (ROW_CHUNKS >= 16) return ((row & 7) << 1) | ((row >> 3) & 1);
  // 128-byte rows: the row parity picks the half of the 256-byte bank period.
  return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}
template <int ROW_CHUNKS>
__device__ __forceinline__ int dkdv4_off(int row, int byte_in_row) {
  const int c = byte_in_row >> 4;
  return row * (ROW_CHUNKS * 16) + (((c ^ dkdv4_swz<ROW_CHUNKS>(row)) << 4) | (byte_in_row & 15));
}

// C += A * B, 16x16 output, K = 32, bf16 operands, fp32 accumulate.
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct Dkdv4Tile {
  static constexpr int NW = 4;
  static constexpr int BKV = 64, BQ = 64;
  static constexpr int ROWB = D * 2, RC = ROWB / 16;
  static constexpr int QTILEB = BQ * ROWB;
  static constexpr int QCPW = QTILEB / (1024 * NW);
  static_assert(QTILEB % (1024 * NW) == 0, "tiles must split evenly");
};

template <int D, bool CAUSAL, bool GF32, bool VARLEN = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dkdv4_kernel(BwdArgs a) {
  using T = Dkdv4Tile<D>;
  constexpr int BKV = T::BKV, BQ = T::BQ, ROWB = T::ROWB, RC = T::RC, QTILEB = T::QTILEB, QCPW = T::QCPW;
  constexpr int NK32 = D / 32, NDB = D / 16;  // 32-wide head-dim steps, 16-wide head-dim blocks

  __shared__ __attribute__((aligned(16))) char sQ0[QTILEB];
  __shared__ __attribute__((aligned(16))) char sQ1[QTILEB];
  __shared__ __attribute__((aligned(16))) char sDO0[QTILEB];
  __shared__ __attribute__((aligned(16))) char sDO1[QTILEB];
  __shared__ __attribute__((aligned(16))) float sL0[BQ];
  __shared__ __attribute__((aligned(16))) float sL1[BQ];
  __shared__ __attribute__((aligned(16))) float sD0[BQ];
  __shared__ __attribute__((aligned(16))) float sD1[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same value, known to be wave-uniform
  const int G = lane >> 4;  // lane group of the 16x16x32 layouts
  const int n16 = lane & 15;

  const UnitItem ui = xcd_decode(blockIdx.x, a.B * a.Hkv);
  const int b = ui.unit / a.Hkv;
  const int hkv = ui.unit % a.Hkv;
  const int kv0 = ui.item * BKV;
  const int key = kv0 + 16 * w + n16;  // this lane's key

  int Nq = a.Nq, Nk = a.Nk;
  size_t kvhead;
  int q_off = 0;
  if constexpr (VARLEN) {
    const SeqSpan sq = clamp_span(a.cu_q[b], a.cu_q[b + 1], a.total_q, a.Nq);
    const SeqSpan sk = clamp_span(a.cu_k[b], a.cu_k[b + 1], a.total_k, a.Nk);
    Nq = sq.len;
    Nk = sk.len;
    if (kv0 >= Nk) return;  // the whole key block lies past this sequence
    q_off = sq.off;
    kvhead = (size_t)hkv * a.total_k + sk.off;
  } else {
    kvhead = (size_t)(b * a.Hkv + hkv) * a.Nk;
  }
  auto q_base = [&](int hq) __attribute__((always_inline)) -> size_t {
    if constexpr (VARLEN) return (size_t)hq * a.total_q + q_off;
    return (size_t)(b * a.Hq + hq) * a.Nq;
  };

  // K and V rows of this lane's key as B operands: head-dim elements
  // 32*kk + 8*G .. +7 (zero past the end of K/V).
  bf16x8 kf[NK32], vf[NK32];
  {
    const bool ok = key < Nk;
    const size_t row = (kvhead + (ok ? key : 0)) * ROWB;
    const char* Kr = (const char*)a.k + row;
    const char* Vr = (const char*)a.v + row;
#pragma unroll
    for (int kk = 0; kk < NK32; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (ok) {
        x = *(const u32x4*)(Kr + (kk * 32 + 8 * G) * 2);
        y = *(const u32x4*)(Vr + (kk * 32 + 8 * G) * 2);
      }
      kf[kk] = __builtin_bit_cast(bf16x8, x);
      vf[kk] = __builtin_bit_cast(bf16x8, y);
    }
  }

  // Per-lane LDS offsets: row reads (row n16 of a 16-row m-block, head-dim
  // step kk) and transpose reads (rows 4G + n16/4 of a 32-row query step,
  // columns of head-dim block db); other m-blocks and query steps are whole
  // 16-row periods away.
  int roff[NK32];
#pragma unroll
  for (int kk = 0; kk < NK32; ++kk) roff[kk] = dkdv4_off<RC>(n16, (kk * 32 + 8 * G) * 2);
  int troff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) troff[db] = dkdv4_off<RC>(4 * G + (n16 >> 2), (db * 16 + 4 * (n16 & 3)) * 2);

  f32x4 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x4{};
    dvacc[db] = f32x4{};
  }

  const int n_qblk = ceil_div(Nq, BQ);
  const int i_first = first_q_tile_for(kv0, BQ, CAUSAL);
  const int n_i = n_qblk - i_first;
  const int total = a.G * n_i;
  const float c = a.c;
  const float scale = a.scale;

  // The next Q block's L and D are loaded into registers (wavefront 0) as
  // its Q/dO tiles are issued and stored to LDS at the end of the current
  // block.
  float lr = 0.0f, dr = 0.0f;
  bool lok = false;
  auto issue_q = [&](int it, char* nQ, char* nDO) __attribute__((always_inline)) {
    const int hm = it / n_i;
    const int i = i_first + it % n_i;
    const int hq = hkv * a.G + hm;
    const size_t qhead = q_base(hq);
    const int q0 = i * BQ;
    if (tid < BQ) {
      lok = q0 + tid < Nq;
      const size_t r = qhead + q0 + (lok ? tid : 0);
      lr = a.lse[r];
      dr = a.dvec[r];
    }
    const char* Qb = uniform_ptr((const char*)a.q + (qhead + q0) * ROWB);
    const char* Ob = uniform_ptr((const char*)a.dout + (qhead + q0) * ROWB);
    const int last = Nq - 1 - q0;
#pragma unroll
    for (int u = 0; u < QCPW; ++u) {
      const int cb = (wu * QCPW + u) * 64;
      const int idx = cb + lane;
      const int row = idx / RC, pc = idx % RC;
      const int lc = pc ^ dkdv4_swz<RC>(row);
      unsigned off = (unsigned)(min(row, last) * ROWB + lc * 16);
      asm volatile("" : "+v"(off));
      load_lds_16(Qb, off, nQ + cb * 16);
      load_lds_16(Ob, off, nDO + cb * 16);
    }
  };
  auto store_ld = [&](float* nL, float* nD) __attribute__((always_inline)) {
    if (tid < BQ) {
      nL[tid] = lok ? lr * kLog2e : INFINITY;
      nD[tid] = lok ? dr : 0.0f;
    }
  };

  if (total > 0) {
    issue_q(0, sQ0, sDO0);
    store_ld(sL0, sD0);
  }
  wait_vmem();
  __syncthreads();

  // One Q block of 64 rows against this wavefront's 16 keys.
  auto body = [&](auto mask_tag, int q0, const char* tQ, const char* tDO, const float* tL, const float* tD)
                  __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // S = Q K^T and dP = dO V^T, m-block mb: queries 16 mb + 4G + i.
    f32x4 s[4], dp[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      s[mb] = f32x4{};
      dp[mb] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < NK32; ++kk) {
        s[mb] = mfma16_bf16(*(const bf16x8*)(tQ + mb * 16 * ROWB + roff[kk]), kf[kk], s[mb]);
        dp[mb] = mfma16_bf16(*(const bf16x8*)(tDO + mb * 16 * ROWB + roff[kk]), vf[kk], dp[mb]);
      }
    }
    // P = exp2(S c - L log2 e), dS = P o (dP - D). Masked: query
    // q0 + 16 mb + 4G + i sees this lane's key iff 16 mb + i >= tq (no query
    // if the key is past the end of K, every query without the causal mask).
    const int tq = key >= Nk ? INT_MAX : (CAUSAL ? key - q0 - 4 * G : INT_MIN);
    float pv[16], dsv[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 lv = *(const f32x4*)(tL + 16 * mb + 4 * G);
      const f32x4 dv = *(const f32x4*)(tD + 16 * mb + 4 * G);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = fast_exp2(fmaf(s[mb][i], c, -lv[i]));
        if constexpr (MASK) p = (16 * mb + i >= tq) ? p : 0.0f;
        pv[4 * mb + i] = p;
        dsv[4 * mb + i] = p * (dp[mb][i] - dv[i]);
      }
    }
    // Query step t: k slots 0-3 hold queries 32t + 4G + i, slots 4-7 hold
    // 32t + 16 + 4G + i (m-blocks 2t and 2t + 1).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pb = to_bf16x8(pv + 8 * t);
      const bf16x8 sb = to_bf16x8(dsv + 8 * t);
      const char* oT = tDO + 32 * t * ROWB;
      const char* qT = tQ + 32 * t * ROWB;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(oT + troff[db]));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(oT + 16 * ROWB + troff[db]));
        dvacc[db] = mfma16_bf16(cat4(lo, hi), pb, dvacc[db]);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(qT + troff[db]));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(qT + 16 * ROWB + troff[db]));
        dkacc[db] = mfma16_bf16(cat4(lo, hi), sb, dkacc[db]);
      }
    }
  };

  auto block = [&](int it, const char* tQ, const char* tDO, const float* tL, const float* tD, char* nQ, char* nDO,
                   float* nL, float* nD) __attribute__((always_inline)) {
    const int i = i_first + it % n_i;
    const int q0 = i * BQ;
    const bool has_next = it + 1 < total;
    if (has_next) issue_q(it + 1, nQ, nDO);
    // Skipped when all of this wavefront's keys lie after all the block's
    // queries; masked when some key lies after some query or past the end.
    const bool active = !CAUSAL || kv0 + 16 * w <= q0 + BQ - 1;
    if (active) {
      const bool need_mask = (CAUSAL && kv0 + 16 * w + 15 > q0) || (kv0 + 16 * w + 16 > Nk);
      if (need_mask)
        body(std::true_type{}, q0, tQ, tDO, tL, tD);
      else
        body(std::false_type{}, q0, tQ, tDO, tL, tD);
    }
    if (has_next) store_ld(nL, nD);
    wait_vmem();
    __syncthreads();
  };
  for (int it = 0; it < total; it += 2) {
    block(it, sQ0, sDO0, sL0, sD0, sQ1, sDO1, sL1, sD1);
    if (it + 1 >= total) break;
    block(it + 1, sQ1, sDO1, sL1, sD1, sQ0, sDO0, sL0, sD0);
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T: head-dim 16 db + 4G + i ----
  if (key < Nk) {
    const size_t rowoff = (kvhead + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d0 = db * 16 + 4 * G;
      const f32x4 kv = {scale * dkacc[db][0], scale * dkacc[db][1], scale * dkacc[db][2], scale * dkacc[db][3]};
      const f32x4 vv = dvacc[db];
      if constexpr (GF32) {
        *(f32x4*)((float*)a.dk + rowoff + d0) = kv;
        *(f32x4*)((float*)a.dv + rowoff + d0) = vv;
      } else {
        *(bf16x4*)((__bf16*)a.dk + rowoff + d0) = __builtin_convertvector(kv, bf16x4);
        *(bf16x4*)((__bf16*)a.dv + rowoff + d0) = __builtin_convertvector(vv, bf16x4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// second pass: dQ_i = scale * sum_j dS_ij K_j, Q-outer like the forward
// ---------------------------------------------------------------------------
//
// The alternative to atomic dQ that page 6.2 section 7.2 names: each
// workgroup owns one Q tile (4 wavefronts x 32 rows, B_r = 128) and walks the
// K/V tiles up to the diagonal, recomputing S, P, dP and dS, so dQ is summed in
// registers and written once (no atomics, no zeroing, deterministic). As in
// the forward, the products are transposed so that each lane owns one query:
// S^T = K Q^T and dP^T = V dO^T take Q and dO as register B operands, L and D
// are per-lane scalars, and dQ^T += K^T dS^T takes dS^T straight from the
// accumulator registers and K^T by transpose reads of the K tile.
// HILO: dS enters the dQ product as a bf16 pair hi + lo (two products, see
// bf16_residual8) instead of one bf16 rounding.
template <int D, bool CAUSAL, bool VARLEN = false, int NW = 4, bool HILO = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = 32 * NW, BC = 64, NKB = BC / 32;
  constexpr int ROWB = D * 2, RC = ROWB / 16, TILEB = BC * ROWB, CPW = TILEB / (1024 * NW);
  constexpr int NKK = D / 16, NDB = D / 32;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole wave loads");

  __shared__ __attribute__((aligned(16))) char sK0[TILEB];
  __shared__ __attribute__((aligned(16))) char sV0[TILEB];
  __shared__ __attribute__((aligned(16))) char sK1[TILEB];
  __shared__ __attribute__((aligned(16))) char sV1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same value, known to be wave-uniform
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int j16 = lane & 15;

  const int n_q_tiles = ceil_div(a.Nq, BR);
  const UnitItem ui = xcd_decode(blockIdx.x, a.B * a.Hkv);
  const int b = ui.unit / a.Hkv;
  const int hkv = ui.unit % a.Hkv;
  const int rank = ui.item / a.G;
  const int hq = hkv * a.G + ui.item % a.G;
  const int qt = CAUSAL ? (n_q_tiles - 1 - rank) : rank;
  const int q0 = qt * BR;
  const int q0w = q0 + 32 * w;
  const int qrow = q0w + l32;

  // Fixed-length [B][H][N][d], or a packed variable-length batch [H][total][d]
  // (a.Nq / a.Nk are then the longest lengths).
  int Nq = a.Nq, Nk = a.Nk;
  size_t qhead, kvhead;
  if constexpr (VARLEN) {
    const SeqSpan sq = clamp_span(a.cu_q[b], a.cu_q[b + 1], a.total_q, a.Nq);
    const SeqSpan sk = clamp_span(a.cu_k[b], a.cu_k[b + 1], a.total_k, a.Nk);
    Nq = sq.len;
    Nk = sk.len;
    if (q0 >= Nq) return;  // the whole Q tile lies past this sequence
    qhead = (size_t)hq * a.total_q + sq.off;
    kvhead = (size_t)hkv * a.total_k + sk.off;
  } else {
    qhead = (size_t)(b * a.Hq + hq) * a.Nq;
    kvhead = (size_t)(b * a.Hkv + hkv) * a.Nk;
  }
  const char* __restrict__ Kh = (const char*)a.k + kvhead * ROWB;
  const char* __restrict__ Vh = (const char*)a.v + kvhead * ROWB;

  bf16x8 qf[NKK], dof[NKK];
  {
    const char* Qr = (const char*)a.q + (qhead + qrow) * ROWB;
    const char* Or = (const char*)a.dout + (qhead + qrow) * ROWB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (qrow < Nq) {
        x = *(const u32x4*)(Qr + (kk * 16 + 8 * g) * 2);
        y = *(const u32x4*)(Or + (kk * 16 + 8 * g) * 2);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, x);
      dof[kk] = __builtin_bit_cast(bf16x8, y);
    }
  }
  // Rows past the end get L = +inf, so their P (and dS) is 0.
  const float l2 = qrow < Nq ? a.lse[qhead + qrow] * kLog2e : INFINITY;
  // D = rowsum(dO o O) of this lane's row (page 6.2, section 7.3), formed
  // here from the dO fragments already in registers and the same head-dim
  // ranges of O (half a row per lane, the other half in lane l ^ 32), and
  // stored for the dK/dV pass, which runs after this one. Rows past the end
  // get D = 0 and store nothing.
  float dq_d = 0.0f;
  {
    float acc = 0.0f;
    if (qrow < Nq) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const f32x8 df = __builtin_convertvector(dof[kk], f32x8);
        f32x8 of;
        if (a.o_f32) {
          const float* Orow = (const float*)a.o + (qhead + qrow) * D + kk * 16 + 8 * g;
          const f32x4 lo = *(const f32x4*)Orow;
          const f32x4 hi = *(const f32x4*)(Orow + 4);
          of = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          const u32x4 ov = *(const u32x4*)((const __bf16*)a.o + (qhead + qrow) * D + kk * 16 + 8 * g);
          of = __builtin_convertvector(__builtin_bit_cast(bf16x8, ov), f32x8);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(df[e], of[e], acc);
      }
    }
    dq_d = half_swap_add(acc);
    if (qrow < Nq && g == 0) a.dvec[qhead + qrow] = dq_d;
  }

  const int kv_end = kv_end_for(q0, BR, Nk, CAUSAL);
  const int n_kv = ceil_div(kv_end, BC);

  // This lane's 16-byte chunk of wave load u of a K/V tile, as a byte offset
  // from the tile's first row. A wave load covers 64 / RC rows; NP loads span
  // the 16-row swizzle period, so NP offsets cover every load of a full tile
  // (load u adds whole periods to offset u % NP); only a ragged last tile
  // recomputes them with the clamp.
  constexpr int RPL = 64 / RC;
  constexpr int NP = (16 / RPL < CPW) ? 16 / RPL : CPW;
  static_assert(CPW % NP == 0 && (CPW == NP || (NP * RPL) % 16 == 0), "wave loads must tile whole swizzle periods");
  int ldoff[NP];
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int idx = (wu * CPW + h) * 64 + lane;
    const int row = idx / RC;
    ldoff[h] = row * ROWB + (((idx % RC) ^ swz<RC>(row)) << 4);
  }
  auto issue_tile = [&](int jt, char* Kt, char* Vt) __attribute__((always_inline)) {
    const int kv0 = jt * BC;
    const char* Kb = uniform_ptr(Kh + (size_t)kv0 * ROWB);
    const char* Vb = uniform_ptr(Vh + (size_t)kv0 * ROWB);
    if (kv0 + BC <= Nk) {
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int cb = (wu * CPW + u) * 64;
        const unsigned off = (unsigned)(ldoff[u % NP] + (u / NP) * NP * RPL * ROWB);
        load_lds_16(Kb, off, Kt + cb * 16);
        load_lds_16(Vb, off, Vt + cb * 16);
      }
    } else {
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int cb = (wu * CPW + u) * 64;
        const int idx = cb + lane;
        const int row = idx / RC, pc = idx % RC;
        const int lc = pc ^ swz<RC>(row);
        const unsigned off = (unsigned)(min(row, Nk - 1 - kv0) * ROWB + lc * 16);
        load_lds_16(Kb, off, Kt + cb * 16);
        load_lds_16(Vb, off, Vt + cb * 16);
      }
    }
  };

  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = tile_off<RC>(l32, (kk * 16 + 8 * g) * 2);
  int troff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      troff[db][h] = tile_off<RC>(4 * g + 8 * h + (j16 >> 2), (db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};
  const float c = a.c;
  // Last key this lane's query row may see (rows past the end of Q are
  // computed like the last row and not stored).
  const int last_key = CAUSAL ? min(qrow, Nk - 1) : Nk - 1;

  // One K/V tile, 32 keys at a time (block kb): S^T and dP^T for the block,
  // then dS^T, then its share of dQ^T += K^T dS^T, so only one block's S^T,
  // dP^T and dS^T are live at once.
  auto body = [&](auto mask_tag, int jt, const char* Kt, const char* Vt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kv0 = jt * BC;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      if constexpr (CAUSAL && NW == 4) {
        // K and V operands of step kk + 2 read before the products of step
        // kk, order pinned (left alone the compiler reads each pair just
        // before its products and waits for it): +1-2 % on causal d = 128
        // backward shapes up to 4K keys; the 8-wavefront instance (-0.6 %)
        // and the non-causal ones (which then spill) keep the plain order.
        constexpr int AH = 2;
        bf16x8 ka[AH + 1], va[AH + 1];
#pragma unroll
        for (int kk = 0; kk < AH; ++kk) {
          ka[kk] = *(const bf16x8*)(Kt + koff[kk] + kb * 32 * ROWB);
          va[kk] = *(const bf16x8*)(Vt + koff[kk] + kb * 32 * ROWB);
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (kk + AH < NKK) {
            ka[(kk + AH) % (AH + 1)] = *(const bf16x8*)(Kt + koff[kk + AH] + kb * 32 * ROWB);
            va[(kk + AH) % (AH + 1)] = *(const bf16x8*)(Vt + koff[kk + AH] + kb * 32 * ROWB);
          }
          sacc = mfma_bf16(ka[kk % (AH + 1)], qf[kk], sacc);
          dpacc = mfma_bf16(va[kk % (AH + 1)], dof[kk], dpacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (kk + AH < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc = mfma_bf16(*(const bf16x8*)(Kt + koff[kk] + kb * 32 * ROWB), qf[kk], sacc);
          dpacc = mfma_bf16(*(const bf16x8*)(Vt + koff[kk] + kb * 32 * ROWB), dof[kk], dpacc);
        }
      }
      // P^T = exp2(S^T c - L log2 e), dS^T = P^T o (dP^T - D)
      // Masked: key kv0 + kb*32 + 8*(r/4) + 4g + r%4 is visible iff it is at
      // most last_key, i.e. iff 8*(r/4) + r%4 <= tk.
      const int tk = last_key - kv0 - kb * 32 - 4 * g;
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(sacc[r], c, -l2));
        if constexpr (MASK) p = (8 * (r >> 2) + (r & 3) <= tk) ? p : 0.0f;
        dsv[r] = p * (dpacc[r] - dq_d);
      }
      // dQ^T += K^T dS^T: slot (g, v) of step t holds key 16t + 8*(v/4) + 4g + v%4
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const bf16x8 sb = to_bf16x8(dsv + 8 * th);
        bf16x8 sl;
        if constexpr (HILO) sl = bf16_residual8(dsv + 8 * th, sb);
        const int t = 2 * kb + th;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* kp = Kt + 16 * t * ROWB;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(kp + troff[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(kp + troff[db][1]));
          dqacc[db] = mfma_bf16(cat4(lo, hi), sb, dqacc[db]);
          if constexpr (HILO) dqacc[db] = mfma_bf16(cat4(lo, hi), sl, dqacc[db]);
        }
      }
      // Keep the next block's operand reads from being hoisted into this one
      // (they would double the live operand registers).
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A step computes tile jt while tile jt+1 streams in. The generic step
  // skips tiles entirely above a wavefront's rows and masks tiles that cross
  // the diagonal or the end of K/V; as in the forward, every tile before the
  // last BR / BC ones is unmasked for every wavefront (Q tiles start at
  // multiples of BR), so the non-causal main loop runs the unmasked body only.
  auto step = [&](auto generic_tag, int jt, const char* Kt, const char* Vt, char* Kn, char* Vn)
                  __attribute__((always_inline)) {
    constexpr bool GENERIC = decltype(generic_tag)::value;
    const int kv0 = jt * BC;
    if (jt + 1 < n_kv) issue_tile(jt + 1, Kn, Vn);
    if constexpr (GENERIC) {
      const bool active = !CAUSAL || kv0 <= q0w + 31;
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > q0w) || (kv0 + BC > Nk);
      if (active) {
        if (need_mask)
          body(std::true_type{}, jt, Kt, Vt);
        else
          body(std::false_type{}, jt, Kt, Vt);
      }
    } else {
      body(std::false_type{}, jt, Kt, Vt);
    }
    wait_vmem();
    __syncthreads();
  };

  // A sequence with no keys (variable-length batches only) has dQ = 0.
  if (n_kv > 0) issue_tile(0, sK0, sV0);
  wait_vmem();
  __syncthreads();
  int jt = 0;
  if constexpr (CAUSAL) {
    // Causal: every step takes the generic form (measured: splitting off the
    // unmasked steps costs more registers than it saves here).
    for (; jt + 1 < n_kv; jt += 2) {
      step(std::true_type{}, jt, sK0, sV0, sK1, sV1);
      step(std::true_type{}, jt + 1, sK1, sV1, sK0, sV0);
    }
    if (jt < n_kv) step(std::true_type{}, jt, sK0, sV0, sK1, sV1);
  } else {
    constexpr int NTAIL = BR / BC;
    const int n_main = n_kv > NTAIL ? n_kv - NTAIL : 0;
    for (; jt + 1 < n_main; jt += 2) {
      step(std::false_type{}, jt, sK0, sV0, sK1, sV1);
      step(std::false_type{}, jt + 1, sK1, sV1, sK0, sV0);
    }
    for (; jt < n_kv; ++jt) {
      if (jt & 1)
        step(std::true_type{}, jt, sK1, sV1, sK0, sV0);
      else
        step(std::true_type{}, jt, sK0, sV0, sK1, sV1);
    }
  }

  if (qrow < Nq) {
    float* dqr = a.dq + (qhead + qrow) * D;
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 v = {scale * dqacc[db][4 * a4], scale * dqacc[db][4 * a4 + 1], scale * dqacc[db][4 * a4 + 2],
                         scale * dqacc[db][4 * a4 + 3]};
        *(f32x4*)(dqr + db * 32 + 8 * a4 + 4 * g) = v;
      }
  }
}

template <int D, bool CAUSAL, bool GF32, bool ATOMIC_DQ>
static hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream) {
  using T = BwdTile<D>;
  constexpr int lds = ATOMIC_DQ ? T::LDS_BYTES_ATOMIC : T::LDS_BYTES_SPLIT;
  auto kern = bwd_kernel<D, CAUSAL, GF32, ATOMIC_DQ>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const long long blocks = (long long)a.B * a.Hkv * ceil_div(a.Nk, T::BKV);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(T::NT), lds, stream, a);
  return hipGetLastError();
}

// The dK/dV pass: at d = 64 the four-wavefront kernel (2-16 % faster on
// MI355X over causal, GQA and non-causal shapes up to 8K keys, level at 16K
// non-causal), else, and with HILO, the eight-wavefront kernel with the P/dS
// exchange (at d = 128 the four-wavefront layout reads 1.6x the LDS bytes
// per flop). At d = 128 the four-wavefront kernel still serves short causal
// rows without query-head groups, where its two independent workgroups per
// CU outweigh the LDS bytes: whole backward +5 % at 1024 keys and +9-12 % at
// 512, but -1 to -2 % at 2048 and -6 % at 4096.
constexpr int kDkdv4MaxKeysD128 = 1024;

template <int D, bool CAUSAL, bool GF32, bool HILO>
static hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  if constexpr (!HILO) {
    if (D == 64 || (CAUSAL && a.G == 1 && a.Nk <= kDkdv4MaxKeysD128)) {
      const long long blocks = (long long)a.B * a.Hkv * ceil_div(a.Nk, Dkdv4Tile<D>::BKV);
      hipLaunchKernelGGL((bwd_dkdv4_kernel<D, CAUSAL, GF32, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
      return hipGetLastError();
    }
  }
  using T = DkdvTile<D, HILO>;
  auto kern = bwd_dkdv_kernel<D, CAUSAL, GF32, false, HILO>;
  const long long blocks = (long long)a.B * a.Hkv * ceil_div(a.Nk, T::BKV);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * T::NW), 0, stream, a);
  return hipGetLastError();
}

// At d = 128 the dQ pass runs with 8 wavefronts (256-row Q tiles sharing
// each K/V tile, one workgroup per CU) from this many keys on. Measured on
// MI355X against 4 wavefronts, whole backward: +1.0-1.8 % at 8K keys,
// +1.7-4.1 % at 16K-32K (causal and not, MHA and GQA), -0.5 to +1.3 % at
// 4K; at d = 64 within +-1 % at 16K, so d = 64 keeps 4 wavefronts.
constexpr int kDq8MinKeys = 8192;

template <int D, bool CAUSAL, bool HILO>
static hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  if constexpr (D == 128) {
    if (a.Nk >= kDq8MinKeys) {
      const long long blocks8 = (long long)a.B * a.Hq * ceil_div(a.Nq, 256);
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, false, 8, HILO>), dim3((unsigned)blocks8), dim3(512), 0, stream,
                         a);
      return hipGetLastError();
    }
  }
  const long long blocks = (long long)a.B * a.Hq * ceil_div(a.Nq, 128);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, false, 4, HILO>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Two-pass backward (fa_bwd): the dQ pass first, which also forms D and
// stores it, then the dK/dV pass, which reads D. The single-pass atomic
// backward (fa_bwd_atomic) keeps the separate preprocess kernel, which also
// zeroes its dQ accumulator.
template <int D, bool CAUSAL, bool GF32>
static hipError_t launch_bwd_all(const BwdArgs& a0, bool o_f32, bool atomic_dq, bool hilo, hipStream_t s) {
  BwdArgs a = a0;
  a.o_f32 = o_f32 ? 1 : 0;
  if (atomic_dq) {
    const long long rows = (long long)a.B * a.Hq * a.Nq;
    const long long threads = rows * (D / 8);
    const unsigned pblocks = (unsigned)((threads + 255) / 256);
    const __bf16* dout = (const __bf16*)a.dout;
    if (o_f32)
      hipLaunchKernelGGL((bwd_preprocess_kernel<D, true, true>), dim3(pblocks), dim3(256), 0, s, dout, a.o, a.dvec, a.dq, rows);
    else
      hipLaunchKernelGGL((bwd_preprocess_kernel<D, false, true>), dim3(pblocks), dim3(256), 0, s, dout, a.o, a.dvec, a.dq, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwd_main<D, CAUSAL, GF32, true>(a, s);
  }
  if (hilo) {
    hipError_t e = launch_bwd_dq<D, CAUSAL, true>(a, s);
    if (e != hipSuccess) return e;
    return launch_bwd_dkdv<D, CAUSAL, GF32, true>(a, s);
  }
  hipError_t e = launch_bwd_dq<D, CAUSAL, false>(a, s);
  if (e != hipSuccess) return e;
  return launch_bwd_dkdv<D, CAUSAL, GF32, false>(a, s);
}

// Packed variable-length batch: the dQ pass (which forms and stores D) and
// then the dK/dV pass; both grids cover the longest sequence and workgroups
// past their sequence's end exit at once. Rows of D that belong to no
// sequence are never read.
template <int D, bool CAUSAL, bool GF32, bool HILO>
static hipError_t launch_bwd_varlen_h(const BwdArgs& a0, bool o_f32, hipStream_t s) {
  BwdArgs a = a0;
  a.o_f32 = o_f32 ? 1 : 0;
  {
    const long long blocks = (long long)a.B * a.Hq * ceil_div(a.Nq, 128);
    if (blocks > 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, true, 4, HILO>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if constexpr (!HILO && D == 64) {
    const long long blocks = (long long)a.B * a.Hkv * ceil_div(a.Nk, Dkdv4Tile<D>::BKV);
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_dkdv4_kernel<D, CAUSAL, GF32, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  using T = DkdvTile<D, HILO>;
  auto kern = bwd_dkdv_kernel<D, CAUSAL, GF32, true, HILO>;
  const long long blocks = (long long)a.B * a.Hkv * ceil_div(a.Nk, T::BKV);
  if (blocks > 0) hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * T::NW), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool GF32>
static hipError_t launch_bwd_varlen_t(const BwdArgs& a, bool o_f32, bool hilo, hipStream_t s) {
  return hilo ? launch_bwd_varlen_h<D, CAUSAL, GF32, true>(a, o_f32, s)
              : launch_bwd_varlen_h<D, CAUSAL, GF32, false>(a, o_f32, s);
}

hipError_t launch_bwd_varlen(const BwdArgs& a, int head_dim, bool causal, bool o_f32, bool grad_f32, bool hilo,
                             hipStream_t s) {
  if (head_dim == 64) {
    if (causal)
      return grad_f32 ? launch_bwd_varlen_t<64, true, true>(a, o_f32, hilo, s)
                      : launch_bwd_varlen_t<64, true, false>(a, o_f32, hilo, s);
    return grad_f32 ? launch_bwd_varlen_t<64, false, true>(a, o_f32, hilo, s)
                    : launch_bwd_varlen_t<64, false, false>(a, o_f32, hilo, s);
  }
  if (causal)
    return grad_f32 ? launch_bwd_varlen_t<128, true, true>(a, o_f32, hilo, s)
                    : launch_bwd_varlen_t<128, true, false>(a, o_f32, hilo, s);
  return grad_f32 ? launch_bwd_varlen_t<128, false, true>(a, o_f32, hilo, s)
                  : launch_bwd_varlen_t<128, false, false>(a, o_f32, hilo, s);
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, bool o_f32, bool grad_f32, bool atomic_dq, bool hilo,
                               hipStream_t s) {
  if (causal)
    return grad_f32 ? launch_bwd_all<D, true, true>(a, o_f32, atomic_dq, hilo, s)
                    : launch_bwd_all<D, true, false>(a, o_f32, atomic_dq, hilo, s);
  return grad_f32 ? launch_bwd_all<D, false, true>(a, o_f32, atomic_dq, hilo, s)
                  : launch_bwd_all<D, false, false>(a, o_f32, atomic_dq, hilo, s);
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool causal, bool o_f32, bool grad_f32, bool atomic_dq,
                      bool hilo, hipStream_t s) {
  return head_dim == 64 ? launch_bwd_d<64>(a, causal, o_f32, grad_f32, atomic_dq, hilo, s)
                        : launch_bwd_d<128>(a, causal, o_f32, grad_f32, atomic_dq, hilo, s);
}

// ---------------------------------------------------------------------------
// scratch for fa_bwd_noalloc
// ---------------------------------------------------------------------------
//
// D = rowsum(dO o O) of fa_bwd_noalloc lives here instead of in a caller's
// workspace: a file-scope device array, one copy per device, held until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol); the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and is kept per device. Every fa_bwd_noalloc call on a device shares that
// device's array: calls that overlap on one device race.
static __device__ __align__(256) float scratch[kBwdNoallocMaxRows];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
}  // namespace

hipError_t bwd_noalloc_scratch(float** dvec) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);  // the same address if two threads race here
  }
  *dvec = p;
  return hipSuccess;
}

}  // namespace fa
