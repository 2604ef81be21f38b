// fa_tiles.h — tile bookkeeping shared by the host code, the host tests and
// the kernels (constexpr, so clang compiles it for both sides).
//
// Causal block classes (page "6.2 FlashAttention V2 chi tiết", section 5.3):
// for a Q tile covering query rows [q0, q0 + nq) and a K/V tile covering key
// columns [k0, k0 + nk),
//   - every entry is visible when the smallest row is at least the largest
//     column (q0 >= k0 + nk - 1): computed without a mask;
//   - every entry is masked when the largest row is below the smallest column
//     (q0 + nq - 1 < k0): the tile is skipped;
//   - otherwise the tile crosses the diagonal and is masked elementwise.
// The inner loop of a causal Q tile therefore stops at
// kv_end = min(N, q0 + nq) (section 6.1).
#pragma once

namespace fa {

enum TileClass : int { kTileFull = 0, kTileDiagonal = 1, kTileSkip = 2 };

constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr TileClass causal_tile_class(int q0, int nq, int k0, int nk) {
  return (q0 + nq - 1 < k0) ? kTileSkip : (q0 >= k0 + nk - 1 ? kTileFull : kTileDiagonal);
}

// One past the last key column a Q tile [q0, q0 + nq) has to visit.
constexpr int kv_end_for(int q0, int nq, int seqlen_k, bool causal) {
  return causal ? (q0 + nq < seqlen_k ? q0 + nq : seqlen_k) : seqlen_k;
}

// Number of K/V tiles of width bc a Q tile visits.
constexpr int kv_tiles_for(int q0, int nq, int seqlen_k, int bc, bool causal) {
  return ceil_div(kv_end_for(q0, nq, seqlen_k, causal), bc);
}

// First Q tile of height br that can see any key of K/V tile [k0, k0 + nk)
// under the causal mask (backward: the Q loop of a K/V column block starts
// at the diagonal).
constexpr int first_q_tile_for(int k0, int br, bool causal) { return causal ? k0 / br : 0; }

// Workgroup -> work-item decode. The work is organised in units (one
// (batch, K/V head) each) of `items` work items, items ordered heaviest
// first. Units vary fastest: all units' first (heaviest) items are dispatched
// first, then all second items, and so on. Workgroups are dispatched
// round-robin over the 8 XCDs of an MI355X (WG L runs on XCD L % 8), so when
// the number of units is a multiple of 8 every workgroup of a unit runs on
// XCD unit % 8 and the unit's K/V stays in that XCD's L2.
// One sequence of a packed variable-length batch: rows [off, off + len) of
// the packed arrays. Built from the caller's cumulative offsets lo = cu[b],
// hi = cu[b + 1], clamped so that a malformed offset array can only give
// wrong rows, never an access outside [0, total) or a length above max_len.
struct SeqSpan {
  int off, len;
};
constexpr SeqSpan clamp_span(int lo, int hi, int total, int max_len) {
  const int o = lo < 0 ? 0 : (lo > total ? total : lo);
  const int e = hi < o ? o : (hi > total ? total : hi);
  const int n = e - o;
  return SeqSpan{o, n < max_len ? n : max_len};
}

struct UnitItem {
  int unit, item;
};
constexpr UnitItem xcd_decode(int L, int units) { return UnitItem{L % units, L / units}; }

}  // namespace fa
