// gfx950 matrix-core building blocks used by the bf16 attention kernels.
//
// v_mfma_f32_32x32x16_bf16, wave64.  Lane l holds
//   A (32 x 16, M x K): row l % 32, k = 8 * (l / 32) + s in slot s = 0..7
//   B (16 x 32, K x N): col l % 32, k = 8 * (l / 32) + s in slot s
//   C (32 x 32):        col l % 32, row 8 * (i / 4) + 4 * (l / 32) + (i % 4) in reg i
// (checked on the hardware).  Only the pairing of A and B slots matters for
// a contraction, so operands may assign any key order to (l / 32, s) as long
// as both sides use the same one.
//
// ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes,
// lane i receives in slot s the 16-bit element i % 4 of the 8 bytes addressed
// by lane 4 * s + i / 4 of its group.  Pointing lane 4 * s + m at
// &X[row_s][col0 + 4 * m] of a row-major tile therefore hands lane i the
// elements X[row_s][col0 + i] for s = 0..3: a column-major operand read
// straight from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
// four words held as one native vector (kept in registers where an array of a
// 16-byte struct copied by value can go to scratch)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// HBM -> LDS copies of 16 bytes per lane through a buffer resource: the
// tile's base address and its size in bytes sit in the (uniform) resource and
// each lane's byte offset in one register, so a copy costs no per-lane 64-bit
// address arithmetic.  A lane whose offset is at or past the size reads zeros.
// (The resource's last word is the raw 32-bit-format value for gfx9-family
// chips.)
typedef __attribute__((address_space(3))) void lds_void_t;
// base and bytes must be the same on every lane; they are read from the first
// lane, so that the resource is built in scalar registers (a resource the
// compiler cannot prove uniform costs a loop over the lanes at every copy).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Physical 16-byte chunk of logical chunk c (0..15) in row r of an LDS tile
// with 256-byte rows (64 bf16): c ^ (4 (r % 4) + (r / 4) % 4).  A 256-byte
// row spans all 64 banks, so only the chunk positions decide conflicts.  A
// 16-byte row read serves 16 lanes per cycle, 16 consecutive rows at one
// logical chunk: the XOR term runs through all 16 values over r % 16.  A
// transpose read (ds_read_b64_tr_b16) serves 32 lanes per cycle, 4
// consecutive rows (from a multiple of 4) times the 4 chunks of one aligned
// group of 4: the term's high half r % 4 sends the 4 rows to 4 different
// groups.  Measured on gfx950 with the LDS bank-conflict counter: no
// conflict cycles for either (c ^ (2 (r % 8) + (r / 8) % 2) takes twice the
// cycles on the transposes, c ^ (r % 16) four times).
__device__ __forceinline__ int swz256(int r, int c) { return c ^ (((r & 3) << 2) | ((r >> 2) & 3)); }
// The same for 128-byte rows (32 bf16, 8 chunks), which cover half the banks:
// even rows one half, odd rows the other.  c ^ (4 ((r / 2) % 2) + (r / 4) % 4)
// gives the 8 rows of one parity among 16 consecutive rows 8 different chunks
// (row reads), and rows 4a and 4a + 2 (4a + 1 and 4a + 3) different groups of
// 4 (transposes).  Measured the same way: no conflict cycles, where c ^ (r % 8)
// takes twice the cycles on both.
__device__ __forceinline__ int swz128(int r, int c) { return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)); }

// Two transpose reads (slots 0..3 from p0, 4..7 from p1) as one operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_read8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// x as three bf16 terms t0 + t1 + t2 (t0 = bf16(x), t1 = bf16(x - t0),
// t2 = bf16(x - t0 - t1); the residuals are exact in fp32, so the sum equals
// x up to 2^-24 |x|), packed {t0 | t1 << 16, t2}.  Against ones in the same
// k-slots of the other operand, one matrix product adds x to every element.
__device__ __forceinline__ uint2 split3_bf16(float x) {
  const float t0 = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
  const float r1 = x - t0;
  const float t1 = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
  const float t2 = __uint_as_float(pack_bf16x2(r1 - t1, 0.f) << 16);
  return make_uint2(pack_bf16x2(t0, t1), pack_bf16x2(t2, 0.f));
}

// Eight fp32 values -> one bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(float x0, float x1, float x2, float x3, float x4,
                                            float x5, float x6, float x7) {
  uint4 u;
  u.x = pack_bf16x2(x0, x1);
  u.y = pack_bf16x2(x2, x3);
  u.z = pack_bf16x2(x4, x5);
  u.w = pack_bf16x2(x6, x7);
  return __builtin_bit_cast(bf16x8, u);
}

// Eight fp32 weights -> one bf16 operand (round to nearest even), adding the
// rounded values to `sum`: a softmax row sum built this way counts exactly
// the weights that the matrix product with V uses, so the normalised output
// is a true weighted mean of the value rows (a lone key gives its value row).
__device__ __forceinline__ bf16x8 to_bf16x8_sum(float x0, float x1, float x2, float x3, float x4, float x5,
                                                float x6, float x7, float& sum) {
  uint4 u;
  u.x = pack_bf16x2(x0, x1);
  u.y = pack_bf16x2(x2, x3);
  u.z = pack_bf16x2(x4, x5);
  u.w = pack_bf16x2(x6, x7);
  // each pair enters the sum through one dot product with (1, 1): the
  // products are the rounded weights themselves, accumulated in fp32
  const bf16x2v one2 = __builtin_bit_cast(bf16x2v, 0x3F803F80u);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w[k]), one2, sum, false);
  return __builtin_bit_cast(bf16x8, u);
}

// Lane l and lane l ^ 32 combined without LDS: v_permlane32_swap exchanges
// the upper half of one copy with the lower half of the other, so the two
// results hold (own, partner) in some order on every lane and their max or
// sum is the pair's, the same in both lanes (both operations commute).
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace ssa
