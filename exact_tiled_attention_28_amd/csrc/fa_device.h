// fa_device.h — gfx950 device helpers shared by the attention kernels:
// vector types, MFMA wrappers, the LDS chunk swizzle, bf16 packing and the
// cross-half-wave exchange used by the row reductions.
//
// MFMA lane layouts used throughout (CDNA3/CDNA4 ISA, 32x32 output blocks):
//   A operand (M x K): lane l holds row m = l % 32 and a set of K values that
//                      depends only on the half-wave g = l / 32;
//   B operand (K x N): lane l holds column n = l % 32 and the same K set;
//   C (M x N, 16 fp32 per lane): lane l holds column n = l % 32 and rows
//                      m = 8 * (r / 4) + 4 * g + (r % 4) for register r.
// A and B use one common (half-wave, element) -> k numbering, so a product
// only needs both operands to put the same k in the same slot; which physical
// k that is does not matter. The kernels use this freedom to feed an
// accumulator straight back as the next product's B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// C += A * B, 32x32 output, K = 16, bf16 operands, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C += A * B, 32x32 output, K = 2, fp32 operands, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value of the same register in lane l ^ 32, combined with op; returns
// op(x[l], x[l ^ 32]) in every lane.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round 8 fp32 values to bf16 (round-to-nearest-even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

// Second half of a two-term bf16 representation x = hi + lo: with hi the RNE
// bf16 rounding of x, x - hi is exact in fp32 (it only holds the low bits of
// x's significand), and lo is its RNE bf16 rounding, so hi + lo carries x to
// a relative error of at most 2^-18 (two products, one per term, replace the
// single bf16 product).
__device__ __forceinline__ bf16x8 bf16_residual8(const float* x, bf16x8 hi) {
  const f32x8 h = __builtin_convertvector(hi, f32x8);
  float r[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) r[v] = x[v] - h[v];
  return to_bf16x8(r);
}

// LDS tiles hold rows of ROW_CHUNKS 16-byte chunks (ROW_CHUNKS = 4, or >= 8
// with rows a multiple of 128 bytes). Chunk c of row r is stored at chunk position
// c ^ swz(r). The gfx950 LDS serves 64 banks of 4 bytes (256 bytes) per
// cycle; swz is chosen so that the two operand reads of the kernels touch
// 64 distinct banks in every cycle:
//  - ds_read_b128 (16 lanes per cycle): 16 consecutive rows, aligned to 16,
//    at one logical chunk must land on 16 distinct 16-byte bank groups;
//  - ds_read_b64_tr_b16 (32 lanes per cycle): 4 consecutive rows, aligned to
//    4, times an aligned block of 4 chunks must land on 16 distinct groups,
//    so the 4 rows must move the block to 4 different blocks.
// 256-byte rows (16 chunks): swz(r) = 4*(r%4) + (r/4)%4 - a bijection on
// r % 16 whose block index (swz / 4) differs across any 4 aligned rows.
// 128-byte rows (8 chunks): two rows share a 256-byte bank period and the
// row parity selects its half; swz(r) = 4*((r/2)%2) + (r/4)%4 is a bijection
// on bits 1-3 of r, and rows r and r+2 of any 4 aligned rows (same parity)
// get different blocks.
// 64-byte rows (4 chunks, the FP8 K tile at d = 64, read only by
// ds_read_b128 of 16 consecutive rows at one logical chunk): four rows share
// a bank period, row % 4 picks the quarter, and swz(r) = (r/4) % 4 gives the
// four rows of one quarter four different chunks.
// swz depends only on r % 16, so moving by whole 16-row steps keeps every
// lane's chunk position; all kernels step their per-lane offsets by multiples
// of 16 rows.
template <int ROW_CHUNKS>
__device__ __forceinline__ int swz(int row) {
  static_assert(ROW_CHUNKS == 4 || ROW_CHUNKS >= 8, "rows of 64 or at least 128 bytes");
  if constexpr (ROW_CHUNKS >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  if constexpr (ROW_CHUNKS == 4) return (row >> 2) & 3;
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of (row, byte-in-row) inside a swizzled LDS tile.
template <int ROW_CHUNKS>
__device__ __forceinline__ int tile_off(int row, int byte_in_row) {
  int c = byte_in_row >> 4;
  return row * (ROW_CHUNKS * 16) + (((c ^ swz<ROW_CHUNKS>(row)) << 4) | (byte_in_row & 15));
}

// Transpose reads of 4 bf16 down a column of a swizzled bf16 LDS tile
// (ds_read_b64_tr_b16, which the kernels issue with per-lane offsets
// computed once): each lane supplies the address of 4 consecutive columns of
// one row; within each 16-lane block the hardware hands lane i element i%4
// of lane 4e + i/4 as its element e (checked on gfx950). With lane j of
// block b pointing at row row_base + j/4, columns col_base + 16*(b%2) +
// 4*(j%4), lane i of block b receives rows row_base + e (e = 0..3) of column
// col_base + 16*(b%2) + i.
//
// Two transpose reads joined into one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 cat4(short4v a, short4v b) {
  typedef __attribute__((ext_vector_type(8))) short short8v;
  short8v r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Word 3 of a raw buffer resource on gfx950 (as on the other gfx9 parts):
// 32-bit data format, no swizzle; with stride 0 the resource is a plain
// byte-addressed range of num_records bytes.
constexpr int kRawBufferWord3 = 0x00020000;

// HBM -> LDS without registers, through a buffer resource
// (buffer_load_dwordx4 ... lds): lane l fetches the 16 bytes at byte offset
// voff from base into lds_wave_base + 16*l. base and lds_wave_base must be
// uniform across the wavefront (base in scalar registers, see uniform_ptr).
// The buffer form rather than global_load_lds_dwordx4: the compiler treats
// the global form as an access that may reach LDS through the flat address
// space and, while one is in flight, waits for every LDS read before using
// any (lgkmcnt(0)); with the buffer form it counts LDS reads in order.
__device__ __forceinline__ void load_lds_16(const char* base, unsigned voff, void* lds_wave_base) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, kRawBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)lds_wave_base, 16, voff, 0, 0, 0);
}

// The same pointer, read from the first active lane into scalar registers
// (the caller guarantees it is wave-uniform). The result is opaque to the
// compiler's loop analysis, so address arithmetic on it is not hoisted into
// per-lane registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t x = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// Wait until this wavefront's outstanding vector-memory loads (including the
// HBM -> LDS ones) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until this wavefront's LDS instructions have completed:
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maximum, no wait).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that orders the compiler's memory accesses around it but
// adds no waits of its own (s_barrier between two compiler memory fences).
// The caller waits for what the other wavefronts must see first: its own
// HBM -> LDS loads (wait_vmem_n) and, before others may overwrite LDS it has
// read, its LDS reads (wait_lds).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wavefront's vector-memory loads are still in
// flight (s_waitcnt vmcnt(N); the counter is 6 bits, split over simm16 bits
// 3:0 and 15:14). Loads retire from the counter in issue order.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace fa
