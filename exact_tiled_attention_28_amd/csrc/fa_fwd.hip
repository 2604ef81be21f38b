// fa_fwd.hip — exact attention forward for gfx950, FlashAttention-2 order.
//
// Method (page "6.2 FlashAttention V2 chi tiết", sections 2.2, 3.2, 4.2, 5.3,
// 6.1; CSDN FlashAttention-2 article, "前向传播" and "工作分区"):
//   * one workgroup per (batch, query head, Q tile of BR rows); the Q tile is
//     read from HBM once and stays in registers for the whole inner loop;
//   * the inner loop streams K/V tiles of BC keys through double-buffered LDS
//     and stops at the causal diagonal;
//   * each wavefront owns 32 query rows of the Q tile and sees the whole K/V
//     tile, so no softmax statistics are merged between wavefronts;
//   * running row max m and row sum l; the output accumulator is left
//     unnormalised and only rescaled by exp(m_old - m_new); one division by l
//     at the end, and only L = m + ln(l) is written besides O;
//   * tiles strictly above the diagonal are never visited; tiles that cross
//     it are masked elementwise.
//
// gfx950 mapping. A wavefront computes S^T = K_j Q_i^T (keys x its 32
// queries) with 32x32 MFMAs, so every lane holds one query column of the
// scores: the row max and row sum are in-register reductions plus one
// exchange between the two half-waves. The same lane layout lets the
// probabilities, packed to bf16, serve directly as the B operand of the
// second product O^T += V_j^T P^T, whose accumulator again keeps one query
// per lane, so the rescale by exp(m_old - m_new) is a per-lane scalar
// multiply. Softmax runs in base 2: scores are scaled by |scale| * log2(e)
// in fp32 after the MFMA, and L is converted back to natural log on store.
// A negative scale is folded into the sign of Q as it is loaded (exact).
//
// The fp32 path instantiates the same template with fp32 operands and the
// 32x32x2 fp32 MFMA, so it checks the tiling logic at fp32 precision.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {

template <bool F32IN, int D, int NW>
struct FwdTile {
  static constexpr int EB = F32IN ? 4 : 2;   // bytes per input element
  static constexpr int BR = 32 * NW;         // query rows per workgroup
  // keys per K/V tile: 128 at d = 64 (measured 2-9 % faster than 64 there: the
  // per-tile barrier, max/rescale test and loop costs are halved per score)
  static constexpr int BC = F32IN ? 32 : (D == 64 ? 128 : 64);
  static constexpr int NKB = BC / 32;        // 32-key blocks per tile
  static constexpr int ROWB = D * EB;        // bytes per K/V row
  static constexpr int RC = ROWB / 16;       // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;    // bytes per K or V tile
  static constexpr int NT = 64 * NW;         // threads per workgroup
  static constexpr int CPW = TILEB / (1024 * NW);  // HBM->LDS loads per wave per tile
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole wave loads");
};

// The accumulator is rescaled only on tiles where some row's running max
// grows; on the other tiles exp(m_old - m_new) = 1 for every row and the
// multiply is skipped. The reference max is always the exact running max, so
// the largest probability of a row is exactly 1 (no bf16 rounding on it),
// as in the eager rescale.

template <bool F32IN, int D, bool CAUSAL, bool OUTF32, int NW, bool VARLEN = false, bool PERSIST = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(F32IN ? 1 : 2, F32IN ? 1 : 2)))
fwd_kernel(FwdArgs a) {
  using T = FwdTile<F32IN, D, NW>;
  constexpr int BR = T::BR, BC = T::BC, NKB = T::NKB, ROWB = T::ROWB, RC = T::RC, TILEB = T::TILEB;
  constexpr int CPW = T::CPW;

  // The d = 128 bf16 one-item-per-workgroup instances keep three K buffers
  // and two V buffers (80 KiB, so two 4-wavefront workgroups still share a
  // CU): K_j is fetched two steps before its scores, V_j one step before its
  // product (measured 1-6 % faster than two of each at d = 128; at d = 64,
  // where one more tile per Q tile takes the masked body, 2-8 % slower on
  // sequences up to 4K). The other instances keep two of each. Every buffer
  // is a separate object so that the compiler can tell that the prefetch
  // into one never aliases the reads of another.
  constexpr bool DEEP = !F32IN && !PERSIST && D == 128;
  __shared__ __attribute__((aligned(16))) char sK0[TILEB];
  __shared__ __attribute__((aligned(16))) char sV0[TILEB];
  __shared__ __attribute__((aligned(16))) char sK1[TILEB];
  __shared__ __attribute__((aligned(16))) char sV1[TILEB];
  __shared__ __attribute__((aligned(16))) char sK2[DEEP ? TILEB : 16];

  const int tid = threadIdx.x;
  int lane = tid & 63;  // lane, g, l32 are only changed by the persistent loop's empty asm
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same value, known to be wave-uniform
  int g = lane >> 5;
  int l32 = lane & 31;

  // One work item L: (batch, query head, Q tile).
  auto run_item = [&](const int L) __attribute__((always_inline)) {
    // Work decode: a unit is one (batch, K/V head); its items are the G query
    // heads x the Q tiles, ordered heaviest causal tile first with the G query
    // heads of a tile next to each other; units vary fastest (xcd_decode).
    const UnitItem ui = xcd_decode(L, a.B * a.Hkv);
    const int b = ui.unit / a.Hkv;
    const int hkv = ui.unit % a.Hkv;
    const int rank = ui.item / a.G;
    const int hq = hkv * a.G + ui.item % a.G;
    const int qt = CAUSAL ? (a.n_q_tiles - 1 - rank) : rank;
    const int q0 = qt * BR;
    const int q0w = q0 + 32 * w;
    const int qrow = q0w + l32;

    // Sequence lengths and head bases: fixed-length [B][H][N][d], or a packed
    // variable-length batch [H][total][d] with sequence b at rows
    // [cu[b], cu[b + 1]) (then a.Nq / a.Nk are the longest lengths).
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
      if (Nk == 0) {
        // No keys: O = 0 and L = -inf (logsumexp of an empty set).
        if (qrow < Nq) {
  #pragma unroll
          for (int d0 = 4 * g; d0 < D; d0 += 8) {
            if constexpr (OUTF32)
              *(f32x4*)((float*)a.o + (qhead + qrow) * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
            else
              *(bf16x4*)((__bf16*)a.o + (qhead + qrow) * D + d0) = bf16x4{};
          }
          if (g == 0) a.lse[qhead + qrow] = -INFINITY;
        }
        return;
      }
    } else {
      qhead = (size_t)(b * a.Hq + hq) * a.Nq;
      kvhead = (size_t)(b * a.Hkv + hkv) * a.Nk;
    }
    // (in scalar registers for the three-buffer loop's scalar-base loads)
    const char* __restrict__ Kh = DEEP ? uniform_ptr((const char*)a.k + kvhead * ROWB) : (const char*)a.k + kvhead * ROWB;
    const char* __restrict__ Vh = DEEP ? uniform_ptr((const char*)a.v + kvhead * ROWB) : (const char*)a.v + kvhead * ROWB;

    // ---- Q fragments (B operand of S^T = K Q^T), loaded once ----------------
    using QFrag = std::conditional_t<F32IN, float, bf16x8>;
    constexpr int NQF = F32IN ? D / 2 : D / 16;
    QFrag qf[NQF];
    if constexpr (F32IN) {
      const float* Qr = (const float*)a.q + (qhead + qrow) * D;
      for (int kk = 0; kk < NQF; ++kk) {
        float x = (qrow < Nq) ? Qr[2 * kk + g] : 0.0f;
        qf[kk] = a.neg ? -x : x;
      }
    } else {
      const char* Qr = (const char*)a.q + (qhead + qrow) * ROWB;
      const unsigned sign = a.neg ? 0x80008000u : 0u;
      for (int kk = 0; kk < NQF; ++kk) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < Nq) x = *(const u32x4*)(Qr + (kk * 16 + 8 * g) * 2);
        x ^= sign;
        qf[kk] = __builtin_bit_cast(bf16x8, x);
      }
    }

    const int kv_end = kv_end_for(q0, BR, Nk, CAUSAL);
    const int n_kv = ceil_div(kv_end, BC);

    // ---- K/V tile staging: HBM -> swizzled LDS, no registers ------------------
    // Wave w fills chunks [64*(w*CPW+u), +64) of each tile; chunk p of row r
    // holds logical chunk p ^ swz(r). Rows past the end of K/V repeat the last
    // row (their scores are masked).
    // This lane's 16-byte chunk of wave load u, as a byte offset from the
    // tile's first row: a wave load covers 64 / RC rows and NP loads span the
    // 16-row swizzle period, so NP offsets cover every load of a full tile;
    // only a ragged last tile recomputes them with the clamp.
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

    // One tile (K or V, from head base Xh) into Xt. Each load is the tile's
    // scalar base plus the lane's 32-bit offset (a buffer load whose resource
    // holds the tile base): the tile base is made opaque, and so is the offset
    // right before its use, so that neither is folded into per-lane 64-bit
    // pointers kept live across the loop. In a tile that runs past the end of
    // K/V, rows past the end read the last row instead (their scores are
    // masked).
    // FULL: the caller knows that the tile lies inside K/V.
    auto issue_one = [&](auto full_tag, int jt, const char* __restrict__ Xh, char* Xt) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
      const int kv0 = jt * BC;
      const char* Xb = uniform_ptr(Xh + (size_t)kv0 * ROWB);
      unsigned o[CPW];
  #pragma unroll
      for (int u = 0; u < CPW; ++u) o[u] = (unsigned)(ldoff[u % NP] + (u / NP) * NP * RPL * ROWB);
      if (!FULL && kv0 + BC > Nk) {
        const unsigned last = (unsigned)(Nk - 1 - kv0);  // last row of K/V in this tile
  #pragma unroll
        for (int u = 0; u < CPW; ++u)
          if (o[u] / ROWB > last) o[u] = last * ROWB + o[u] % ROWB;
      }
  #pragma unroll
      for (int u = 0; u < CPW; ++u) {
        unsigned ou = o[u];
        asm volatile("" : "+v"(ou));
        load_lds_16(Xb, ou, Xt + (wu * CPW + u) * 64 * 16);
      }
    };

    f32x16 oacc[D / 32];
  #pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -INFINITY;  // reference max, log2 units (scaled scores)
    float lsum = 0.0f;    // running sum over this half-wave's keys
    const float c = a.c;  // > 0: a zero scale arrives as the smallest normal float
    // Last key this lane's query row may see (rows past the end of Q are
    // computed like the last row and not stored).
    const int last_key = CAUSAL ? min(qrow, Nk - 1) : Nk - 1;

    // Per-lane LDS byte offsets of the MFMA operand fetches, computed once.
    // The swizzle of a row depends only on the row modulo 8, so moving by
    // whole 32-key blocks or 16-key steps adds a constant that folds into the
    // instruction's immediate offset.
    constexpr int NKOFF = F32IN ? 1 : NQF;
    int koff[NKOFF];
    int voff[F32IN ? 1 : D / 32][2];
    if constexpr (!F32IN) {
  #pragma unroll
      for (int kk = 0; kk < NQF; ++kk) koff[kk] = tile_off<RC>(l32, (kk * 16 + 8 * g) * 2);
      const int j = lane & 15;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db)
  #pragma unroll
        for (int h = 0; h < 2; ++h)
          voff[db][h] = tile_off<RC>(4 * g + 8 * h + (j >> 2), (db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)) * 2);
    }

    // Scores, mask and online softmax of tile jt: on return sacc holds P.
    auto body_s = [&](auto mask_tag, int jt, const char* Kt, f32x16(&sacc)[NKB]) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int kv0 = jt * BC;
      // ---- S^T = K_j Q_i^T ------------------------------------------------------
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16{};
        if constexpr (F32IN) {
          const int krow = kb * 32 + l32;
  #pragma unroll
          for (int kk = 0; kk < NQF; ++kk) {
            const float ka = *(const float*)(Kt + tile_off<RC>(krow, (2 * kk + g) * 4));
            sacc[kb] = mfma_f32(ka, qf[kk], sacc[kb]);
          }
        } else if constexpr (!DEEP) {
  #pragma unroll
          for (int kk = 0; kk < NQF; ++kk) {
            const bf16x8 ka = *(const bf16x8*)(Kt + koff[kk] + kb * 32 * ROWB);
            sacc[kb] = mfma_bf16(ka, qf[kk], sacc[kb]);
          }
        }
      }
      if constexpr (DEEP) {
        // The K operands of step kk + 1 are read before the products of step
        // kk, and the schedule is pinned to that order: left to itself the
        // compiler reads each operand just before its product and waits for
        // it (measured 0.5-3 % slower on d = 128 shapes).
        bf16x8 ka[2][NKB];
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) ka[0][kb] = *(const bf16x8*)(Kt + koff[0] + kb * 32 * ROWB);
  #pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          if (kk + 1 < NQF) {
  #pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              ka[(kk + 1) & 1][kb] = *(const bf16x8*)(Kt + koff[kk + 1] + kb * 32 * ROWB);
          }
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sacc[kb] = mfma_bf16(ka[kk & 1][kb], qf[kk], sacc[kb]);
        }
        // schedule: the first reads, then (next reads, this step's products)
        __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
  #pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          if (kk + 1 < NQF) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NKB, 0);
        }
      }

      // ---- mask (diagonal-crossing or ragged tiles only) ------------------------
      // Key kv0 + kb*32 + 8*(r/4) + 4g + r%4 is visible iff it is at most
      // last_key; with the lane's part folded into t, each test compares a
      // constant with t. Masked scores become -inf, which the exp2 below
      // (multiplier c > 0) turns into probability 0.
      if constexpr (MASK) {
        const int t = last_key - kv0 - 4 * g;
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) <= t) ? sacc[kb][r] : -INFINITY;
      }

      // ---- online softmax ---------------------------------------------------------
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
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      }
      float rs = 0.0f;
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[kb][r], c, -m));
          sacc[kb][r] = p;
          rs += p;
        }
      lsum += rs;
    };

    // O^T += V_j^T P^T for the probabilities in sacc.
    auto body_pv = [&](const char* Vt, f32x16(&sacc)[NKB]) __attribute__((always_inline)) {
      if constexpr (F32IN) {
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
  #pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const float va = *(const float*)(Vt + tile_off<RC>(key, (db * 32 + l32) * 4));
              oacc[db] = mfma_f32(va, sacc[kb][r], oacc[db]);
            }
          }
      } else {
        // Step t covers keys 16t..16t+15; slot (g, v) of both operands holds
        // key 16t + 8*(v/4) + 4g + v%4, which is where the S^T accumulator
        // registers 8*(t%2)..8*(t%2)+7 of block t/2 put it; the V^T operand is
        // read down the key column with two transpose reads.
  #pragma unroll
        for (int t = 0; t < BC / 16; ++t) {
          float pv[8];
  #pragma unroll
          for (int v = 0; v < 8; ++v) pv[v] = sacc[t >> 1][8 * (t & 1) + v];
          const bf16x8 pb = to_bf16x8(pv);
  #pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const char* vp = Vt + 16 * t * ROWB;
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(vp + voff[db][0]));
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS short4v*)(vp + voff[db][1]));
            oacc[db] = mfma_bf16(cat4(lo, hi), pb, oacc[db]);
          }
        }
      }
    };

    auto body = [&](auto mask_tag, int jt, const char* Kt, const char* Vt) __attribute__((always_inline)) {
      f32x16 sacc[NKB];
      body_s(mask_tag, jt, Kt, sacc);
      body_pv(Vt, sacc);
    };

    // A step computes tile jt from (Kt, Vt) while tile jt+1 streams into
    // (Kn, Vn). A wavefront whose 32 rows all lie above the tile skips it;
    // tiles that cross the diagonal or the end of K/V take the masked body.
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

    // Q tiles start at multiples of BR (a multiple of BC), so every tile
    // before the last BR / BC ones ends at or before the first row of the Q
    // tile and inside K/V: it is unmasked for every wavefront, and the main
    // loop runs the unmasked body only. The last BR / BC tiles take the
    // generic step.
    constexpr int NTAIL = BR / BC;
    if constexpr (DEEP) {
      // Loads are issued in the order K_0, V_0, K_1 (here), then V_{j+1},
      // K_{j+2} at the top of step j, into K buffer j % 3 and V buffer j % 2.
      // Step j ends by waiting for K_{j+1} and V_{j+1}: the vector-memory
      // counter retires loads in issue order, so that is "at most the loads
      // of K_{j+2} in flight". The barrier after it makes every wavefront's
      // share of both tiles visible; it also follows the completion of all
      // of the wavefront's LDS reads, so the loads of step j+1 may overwrite
      // V_j and K_j. The barrier is a plain s_barrier between compiler memory
      // fences: a workgroup fence would make the compiler wait for every load
      // in flight. Steps before n_fast are unmasked for every wavefront and
      // have both loads to issue; the others (the last few tiles of a Q
      // tile) check everything and take the masked body.
      // (n_fast also keeps tile j + 2 of a fast step inside K/V)
      const int n_fast = max(0, min(min(n_kv - NTAIL, n_kv - 2), Nk / BC - 2));
      auto dstep = [&](auto generic_tag, int jt, const char* Kt, const char* Vt, char* Vn, char* Kn2)
                       __attribute__((always_inline)) {
        constexpr bool GENERIC = decltype(generic_tag)::value;
        const bool has1 = !GENERIC || jt + 1 < n_kv;
        const bool has2 = !GENERIC || jt + 2 < n_kv;
        if (has1) issue_one(std::bool_constant<!GENERIC>{}, jt + 1, Vh, Vn);
        if (has2) issue_one(std::bool_constant<!GENERIC>{}, jt + 2, Kh, Kn2);
        f32x16 sacc[NKB];
        if constexpr (GENERIC) {
          if (!CAUSAL || jt * BC <= q0w + 31) {
            body_s(std::true_type{}, jt, Kt, sacc);
            body_pv(Vt, sacc);
          }
          if (has2)
            wait_vmem_n<CPW>();
          else
            wait_vmem_n<0>();
        } else {
          body_s(std::false_type{}, jt, Kt, sacc);
          body_pv(Vt, sacc);
          wait_vmem_n<CPW>();
        }
        wait_lds();
        lds_barrier();
      };
      issue_one(std::false_type{}, 0, Kh, sK0);
      issue_one(std::false_type{}, 0, Vh, sV0);
      if (n_kv > 1) {
        issue_one(std::false_type{}, 1, Kh, sK1);
        wait_vmem_n<CPW>();
      } else {
        wait_vmem_n<0>();
      }
      __syncthreads();
      // Main loop: unmasked steps only, unrolled over the six (K buffer,
      // V buffer) phases so that every buffer is a compile-time choice; it
      // can leave after any phase.
      int jt = 0;
      if (n_fast > 0) {
        while (true) {
          dstep(std::false_type{}, jt, sK0, sV0, sV1, sK2);
          if (++jt >= n_fast) break;
          dstep(std::false_type{}, jt, sK1, sV1, sV0, sK0);
          if (++jt >= n_fast) break;
          dstep(std::false_type{}, jt, sK2, sV0, sV1, sK1);
          if (++jt >= n_fast) break;
          dstep(std::false_type{}, jt, sK0, sV1, sV0, sK2);
          if (++jt >= n_fast) break;
          dstep(std::false_type{}, jt, sK1, sV0, sV1, sK0);
          if (++jt >= n_fast) break;
          dstep(std::false_type{}, jt, sK2, sV1, sV0, sK1);
          if (++jt >= n_fast) break;
        }
      }
      // The last few tiles: generic steps, in the phase the main loop left.
      for (; jt < n_kv; ++jt) {
        switch (jt % 6) {
          case 0: dstep(std::true_type{}, jt, sK0, sV0, sV1, sK2); break;
          case 1: dstep(std::true_type{}, jt, sK1, sV1, sV0, sK0); break;
          case 2: dstep(std::true_type{}, jt, sK2, sV0, sV1, sK1); break;
          case 3: dstep(std::true_type{}, jt, sK0, sV1, sV0, sK2); break;
          case 4: dstep(std::true_type{}, jt, sK1, sV0, sV1, sK0); break;
          default: dstep(std::true_type{}, jt, sK2, sV1, sV0, sK1); break;
        }
      }
    } else {
      const int n_main = n_kv > NTAIL ? n_kv - NTAIL : 0;
      issue_tile(0, sK0, sV0);
      wait_vmem();
      __syncthreads();
      int jt = 0;
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

    // ---- epilogue: O = O~ / l, L = m + ln l ------------------------------------
    const float lt = half_swap_add(lsum);
    const float inv = 1.0f / lt;
    if (qrow < Nq) {
      const size_t orow = (qhead + qrow) * D;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db)
  #pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = db * 32 + 8 * a4 + 4 * g;
          f32x4 ov = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                      oacc[db][4 * a4 + 3] * inv};
          if constexpr (OUTF32) {
            *(f32x4*)((float*)a.o + orow + d0) = ov;
          } else {
            *(bf16x4*)((__bf16*)a.o + orow + d0) = __builtin_convertvector(ov, bf16x4);
          }
        }
      if (g == 0) a.lse[qhead + qrow] = (m + fast_log2(lt)) * kLn2;
    }
  };

  if constexpr (!PERSIST) {
    run_item(blockIdx.x);
  } else {
    // Work queue (the persistent causal scheduler of the FlashAttention-3
    // news page, on persistent kernels): the grid holds only as many
    // workgroups as stay resident, and each pulls items until none are
    // left. Item L lives in queue L mod 8, in increasing L, i.e. the same
    // heaviest-first order and the same XCD (workgroup b runs on XCD
    // b mod 8 under round-robin dispatch) as the one-workgroup-per-item
    // grid; a workgroup whose own queue is empty takes the remaining
    // (lightest) items of the other queues. Thread 0 takes its next
    // position in the current queue as an item starts and looks at the
    // answer only when the item is done, so the atomic's latency overlaps
    // the item's first loads; only a queue change waits on the atomics.
    // Counters: sched[0..7] queue positions, sched[8] finished workgroups;
    // the last workgroup to finish sets all nine back to zero, so every
    // launch starts from zeros once the caller has zeroed them before the
    // first launch.
    __shared__ int s_next;
    int* const sched = a.sched;
    const int total = a.B * a.Hq * a.n_q_tiles;
    const int x0 = blockIdx.x & 7;
    int qs = 0;  // queues emptied so far (meaningful in thread 0 only)
    auto fetch_now = [&]() __attribute__((always_inline)) {
      while (qs < 8) {
        const int x = (x0 + qs) & 7;
        const long long L = x + 8LL * atomicAdd(&sched[x], 1);
        if (L >= 0 && L < total) return (int)L;  // out of range (or a counter that was not zero): queue done
        ++qs;
      }
      return -1;
    };
    if (tid == 0) s_next = fetch_now();
    __syncthreads();
    int L = s_next;
    while (L >= 0) {
      int pos = 0;
      if (tid == 0 && qs < 8) pos = atomicAdd(&sched[(x0 + qs) & 7], 1);
      // The lane ids pass through an empty asm once per item, so that the
      // lane-dependent offsets of an item are recomputed per item instead
      // of being hoisted out of this loop and kept live across it.
      asm volatile("" : "+v"(lane), "+v"(g), "+v"(l32));
      run_item(L);  // has at least one barrier before its end: s_next is free
      if (tid == 0) {
        int nl = -1;
        if (qs < 8) {
          const long long cand = ((x0 + qs) & 7) + 8LL * pos;
          nl = (int)cand;
          if (cand < 0 || cand >= total) {
            ++qs;
            nl = fetch_now();
          }
        }
        s_next = nl;
      }
      __syncthreads();
      L = s_next;
    }
    if (tid == 0 && atomicAdd(&sched[8], 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int x = 0; x < 9; ++x) atomicExch(&sched[x], 0);
    }
  }
}

// Causal bf16 input from this many keys on runs fwd_kernel with 8
// wavefronts (256-row Q tiles sharing each K/V tile). Measured on MI355X
// against the 4-wavefront kernel: d = 128 (both with three K buffers) 2 %
// faster at 16K keys, 1.6 % slower at 8K (and 2-14 % slower below 8K with
// two buffers: fewer, longer workgroups balance worse on short causal rows);
// d = 64 3.3-3.4 % faster at 16K, 2.4 % at 32K.
constexpr int kWide8MinKeys = 16384;
// Without the causal mask the 8-wavefront kernel runs from this many keys
// on: measured at d = 128 3.6 % faster at 8K, 5 % at 16K, 2-5 % at 32K (MHA
// and GQA), and with the buffer-form tile loads 4.1 % faster at 4K; at
// d = 64 5 % faster at 8K and 16K, 2.3 % at 32K, 1 % at 4K.
constexpr int kWide8MinKeysNonCausal = 4096;

template <bool F32IN, int D, bool CAUSAL, bool OUTF32>
static hipError_t launch_fwd_t(FwdArgs a, hipStream_t stream) {
  if constexpr (!F32IN) {
    if (a.Nk >= (CAUSAL ? kWide8MinKeys : kWide8MinKeysNonCausal)) {
      using T8 = FwdTile<false, D, 8>;
      a.n_q_tiles = ceil_div(a.Nq, T8::BR);
      const long long blocks8 = (long long)a.B * a.Hq * a.n_q_tiles;
      hipLaunchKernelGGL((fwd_kernel<false, D, CAUSAL, OUTF32, 8>), dim3((unsigned)blocks8), dim3(T8::NT), 0, stream,
                         a);
      return hipGetLastError();
    }
  }
  constexpr int NW = 4;
  using T = FwdTile<F32IN, D, NW>;
  a.n_q_tiles = ceil_div(a.Nq, T::BR);
  const long long blocks = (long long)a.B * a.Hq * a.n_q_tiles;
  hipLaunchKernelGGL((fwd_kernel<F32IN, D, CAUSAL, OUTF32, NW>), dim3((unsigned)blocks), dim3(T::NT), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool OUTF32>
static hipError_t launch_fwd_varlen_t(FwdArgs a, hipStream_t stream) {
  constexpr int NW = 4;
  using T = FwdTile<false, D, NW>;
  a.n_q_tiles = ceil_div(a.Nq, T::BR);
  const long long blocks = (long long)a.B * a.Hq * a.n_q_tiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<false, D, CAUSAL, OUTF32, NW, true>), dim3((unsigned)blocks), dim3(T::NT), 0, stream,
                     a);
  return hipGetLastError();
}

// Resident workgroups of a persistent forward instance on the current device.
template <int D, bool CAUSAL, bool OUTF32>
static int persistent_slots() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&fwd_kernel<false, D, CAUSAL, OUTF32, 4, false, true>), 256, 0) !=
      hipSuccess)
    return 0;
  return cus * per_cu;
}

template <int D, bool CAUSAL, bool OUTF32>
static hipError_t launch_fwd_persistent_t(FwdArgs a, hipStream_t stream) {
  constexpr int NW = 4;
  using T = FwdTile<false, D, NW>;
  a.n_q_tiles = ceil_div(a.Nq, T::BR);
  const long long items = (long long)a.B * a.Hq * a.n_q_tiles;
  const int slots = persistent_slots<D, CAUSAL, OUTF32>();
  if (slots <= 0) return hipErrorInvalidDeviceFunction;
  long long grid = items < slots ? items : slots;
  if (grid >= 8) grid -= grid % 8;  // whole sets of 8, one per XCD
  hipLaunchKernelGGL((fwd_kernel<false, D, CAUSAL, OUTF32, NW, false, true>), dim3((unsigned)grid), dim3(T::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_persistent(const FwdArgs& a, int head_dim, bool causal, bool out_f32, hipStream_t s) {
  if (head_dim == 64) {
    if (causal)
      return out_f32 ? launch_fwd_persistent_t<64, true, true>(a, s) : launch_fwd_persistent_t<64, true, false>(a, s);
    return out_f32 ? launch_fwd_persistent_t<64, false, true>(a, s) : launch_fwd_persistent_t<64, false, false>(a, s);
  }
  if (causal)
    return out_f32 ? launch_fwd_persistent_t<128, true, true>(a, s) : launch_fwd_persistent_t<128, true, false>(a, s);
  return out_f32 ? launch_fwd_persistent_t<128, false, true>(a, s) : launch_fwd_persistent_t<128, false, false>(a, s);
}

hipError_t launch_fwd_varlen(const FwdArgs& a, int head_dim, bool causal, bool out_f32, hipStream_t s) {
  if (head_dim == 64) {
    if (causal) return out_f32 ? launch_fwd_varlen_t<64, true, true>(a, s) : launch_fwd_varlen_t<64, true, false>(a, s);
    return out_f32 ? launch_fwd_varlen_t<64, false, true>(a, s) : launch_fwd_varlen_t<64, false, false>(a, s);
  }
  if (causal) return out_f32 ? launch_fwd_varlen_t<128, true, true>(a, s) : launch_fwd_varlen_t<128, true, false>(a, s);
  return out_f32 ? launch_fwd_varlen_t<128, false, true>(a, s) : launch_fwd_varlen_t<128, false, false>(a, s);
}

template <bool F32IN, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, bool out_f32, hipStream_t s) {
  if (causal) return out_f32 ? launch_fwd_t<F32IN, D, true, true>(a, s) : launch_fwd_t<F32IN, D, true, false>(a, s);
  return out_f32 ? launch_fwd_t<F32IN, D, false, true>(a, s) : launch_fwd_t<F32IN, D, false, false>(a, s);
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool in_f32, bool causal, bool out_f32, hipStream_t s) {
  if (in_f32) {
    return head_dim == 64 ? launch_fwd_d<true, 64>(a, causal, out_f32, s)
                          : launch_fwd_d<true, 128>(a, causal, out_f32, s);
  }
  return head_dim == 64 ? launch_fwd_d<false, 64>(a, causal, out_f32, s)
                        : launch_fwd_d<false, 128>(a, causal, out_f32, s);
}

}  // namespace fa
