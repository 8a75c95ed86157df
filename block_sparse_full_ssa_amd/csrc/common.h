// Device-side helpers shared by the libssa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

constexpr int kWave = 64;

// bf16 is carried as its raw 16 bits; widening to fp32 is a shift.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (gfx950 has a hardware conversion).
__device__ __forceinline__ bf16_t to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, h);
  return r;
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return to_bf16(x); }

// Sum over the 64 lanes of a wave; every lane receives the total.  The
// butterfly order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

// Maximum of an unsigned value over the 64 lanes of a wave, returned to every
// lane: DPP row shifts build prefix maxima within each row of 16 lanes, row
// broadcasts carry them across rows, and lane 63 ends with the total.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, false)));  // row_shr:1
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, false)));  // row_shr:2
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, false)));  // row_shr:4
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, false)));  // row_shr:8
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xa, 0xf, false)));  // row_bcast:15
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xc, 0xf, false)));  // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Order-preserving map of a finite fp32 score to an unsigned integer.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), off, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), off, kWave);
    uint64_t y = (static_cast<uint64_t>(hi) << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

// Work item of a query-stationary grid (one workgroup per query head and
// query tile), from the linear workgroup index L.  Workgroups are dispatched
// round-robin over the eight XCDs (L % 8), each with its own L2.  Where the KV
// heads divide evenly over the XCDs, or the XCDs over the KV heads, all G
// query heads of a KV head run on the same XCD(s), so the K/V tiles they all
// stream fill one L2 instead of up to G of them.  Query tiles go out longest
// first: rank 0 is the last tile.  Results are uniform (scalar registers).
struct QTileItem {
  int bh;      // batch * Hq + query head
  int rank;    // query tile n_qtiles - 1 - rank
};
__device__ __forceinline__ QTileItem qtile_item(int L, int nkv, int G, int nqt) {
  constexpr int X = 8;
  int bh, rank;
  if (nkv % X == 0) {
    const int per = (nkv / X) * G;              // items of one tile rank on an XCD
    const int x = L % X, s = L / X, rem = s % per;
    bh = (x + X * (rem / G)) * G + rem % G;
    rank = s / per;
  } else if (X % nkv == 0 && (G * nqt) % (X / nkv) == 0) {
    const int r = X / nkv;                      // XCDs per KV head
    const int x = L % X;
    const int idx = (L / X) * r + x / nkv;      // item of KV head x % nkv
    bh = (x % nkv) * G + idx % G;
    rank = idx / G;
  } else {
    bh = L % (nkv * G);
    rank = L / (nkv * G);
  }
  return {__builtin_amdgcn_readfirstlane(bh), __builtin_amdgcn_readfirstlane(rank)};
}

}  // namespace ssa
