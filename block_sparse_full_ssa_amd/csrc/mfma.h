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
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace ssa
