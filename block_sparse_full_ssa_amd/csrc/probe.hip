// Machine probes for the measurement harness: a dense bf16 matrix-core loop
// and a plain device copy.  They measure the two ceilings that the attention
// kernels' rates are read against -- the matrix rate the chip sustains under
// full load (its clock then sits below the one the datasheet peak assumes)
// and the HBM bandwidth a streaming kernel reaches.  They compute nothing of
// the attention method.

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kChains = 4;   // independent accumulators per wave

// Each wave runs kChains independent chains of 32x32x16 bf16 products, so
// the matrix pipe never waits on a result; two workgroups per CU put two
// waves on every SIMD, as in the attention kernels.
__global__ void __launch_bounds__(256, 2) k_probe_mfma(float* sink, int iters) {
  const int t = threadIdx.x;
  // operands: small normal bf16 values that depend on the lane
  const uint32_t ua = 0x3c003c00u + ((t & 7) * 0x00010001u);
  const uint32_t ub = 0x3b803b80u + (((t >> 3) & 7) * 0x00010001u);
  const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(ua, ua, ua, ua));
  const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(ub, ub, ub, ub));
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + t] = s;
}

// 16-byte vectors, four loads in flight per lane, grid-stride over the
// whole buffer; the tail (fewer than 4 * 256 vectors per block) is handled
// by the per-vector bound.
__global__ void __launch_bounds__(256) k_probe_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 1024;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x; base < n; base += stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + 256 * u < n) v[u] = src[base + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + 256 * u < n) dst[base + 256 * u] = v[u];
  }
}

}  // namespace

void launch_probe_mfma(float* sink, int blocks, int iters, hipStream_t s) {
  timing_begin(kKProbeMfma, s);
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0, s, sink, iters);
  timing_end(kKProbeMfma, s);
}

void launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  const int64_t want = (n + 1023) / 1024;
  const int blocks = static_cast<int>(want < 4096 ? want : 4096);
  timing_begin(kKProbeCopy, s);
  hipLaunchKernelGGL(k_probe_copy, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  timing_end(kKProbeCopy, s);
}

}  // namespace ssa
