// Machine probes for the measurement harness: a dense bf16 matrix-core loop,
// a plain device copy, fp32 global atomics and LDS operand reads.  They measure the two ceilings that the attention
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

// fp32 global atomics: workgroup w adds 1.0 to every float of 16 KiB tile
// w % ntiles, `iters` times (16 coalesced atomic instructions per wave per
// pass).  The tiles stay resident in the caches, so the time is the rate at
// which the chip performs the atomics themselves.
__global__ void __launch_bounds__(256) k_probe_atomic(float* buf, int ntiles, int iters) {
  float* t = buf + static_cast<int64_t>(blockIdx.x % ntiles) * 4096;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) atomicAdd(&t[r * 256 + threadIdx.x], 1.0f);
  }
}

// LDS reads: every wave reads its own 8 KiB of a 32 KiB tile, eight reads per
// pass, either 16 bytes per lane (ds_read_b128, conflict-free: lane l reads
// chunk l) or 8 bytes per lane as transposes (ds_read_b64_tr_b16, the
// operand reads of the attention kernels); modes 2..9 replay the kernels'
// read patterns on swizzled tiles.  The values are folded into the sink so
// that no read is dropped.
__global__ void __launch_bounds__(256, 2) k_probe_lds(float* sink, int iters, int mode) {
  __shared__ __attribute__((aligned(16))) uint16_t buf[256 * 64];
  const int t = threadIdx.x;
  for (int i = t; i < 256 * 64; i += 256) buf[i] = static_cast<uint16_t>(i * 7);
  __syncthreads();
  const int wave = t >> 6, lane = t & 63;
  uint32_t acc = 0u;
  if (mode == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(buf) + wave * 64 + lane;   // chunk < 256 + 64
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint4 v = p[(r * 256) & 1023];                                    // chunk < 2048
        acc += v.x ^ v.y ^ v.z ^ v.w;
        asm volatile("" : "+v"(acc));
      }
    }
  } else if (mode == 1) {
    const int grp = lane >> 4, li = lane & 15;
    const int row = wave * 16 + grp * 4 + (li >> 2), col = 4 * (li & 3);       // row < 64, col < 16
    const uint16_t* base = buf + row * 64 + col;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * (r & 3)));
        acc += static_cast<uint32_t>(v[0] ^ v[1] ^ v[2] ^ v[3]);
        asm volatile("" : "+v"(acc));
      }
    }
  } else {
    // Modes 2..9: the attention kernels' operand reads of a swizzled tile
    // (rows of 256 bytes, 64 bf16, or of 128 bytes, 32 bf16), whose bank
    // conflicts the LDS conflict counter shows.  Row reads: lane (col, g)
    // reads logical chunk 2 s + g of row 32 (s % 2) + col (16 bytes).
    // Transposes: lane (grp, li) reads half (li % 2) of logical chunk
    // 4 dt + 2 (grp % 2) + (li % 4) / 2 of row 16 st + 4 (grp / 2) + li / 4
    // and of the row 8 below.  Swizzles (physical chunk of logical c in row r):
    //   2: transposes, 256-byte rows, c ^ (2 (r % 8) + (r / 8) % 2)
    //   3: transposes, 256-byte rows, c ^ (4 (r % 4) + (r / 4) % 4)
    //   4: transposes, 256-byte rows, c ^ (r % 16)
    //   5: row reads, 256-byte rows, c ^ (4 (r % 4) + (r / 4) % 4)
    //   6: row reads, 128-byte rows, c ^ (r % 8)
    //   7: row reads, 128-byte rows, c ^ (4 ((r / 2) % 2) + (r / 4) % 4)
    //   8: transposes, 128-byte rows, c ^ (r % 8)
    //   9: transposes, 128-byte rows, c ^ (4 ((r / 2) % 2) + (r / 4) % 4)
    const bool wide = mode <= 5, tr = mode <= 4 || mode >= 8;
    const int rowe = wide ? 128 : 64;                      // elements per row
    auto swz = [&](int r, int c) {
      switch (mode) {
        case 2: return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
        case 4: return c ^ (r & 15);
        case 6: case 8: return c ^ (r & 7);
        case 3: case 5: return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
        default: return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
      }
    };
    const int g = lane >> 5, col = lane & 31, grp = lane >> 4, li = lane & 15;
    int o0[8], o1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (tr) {
        const int st = u >> 2, dt = u & (wide ? 3 : 1);
        const int r0 = 16 * st + 4 * (grp >> 1) + (li >> 2) + (wide ? 0 : 32 * ((u >> 1) & 1));
        const int c = 4 * dt + 2 * (grp & 1) + ((li & 3) >> 1), e = 4 * (li & 1);
        o0[u] = r0 * rowe + 8 * swz(r0, c) + e;
        o1[u] = (r0 + 8) * rowe + 8 * swz(r0 + 8, c) + e;
      } else {
        const int r = 32 * (u & 1) + col, s = (u >> 1) & (wide ? 3 : 1);
        o0[u] = r * rowe + 8 * swz(r, 2 * s + g);
        o1[u] = 0;
      }
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tr) {
          const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + o0[u]));
          const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + o1[u]));
          acc += static_cast<uint32_t>(a[0] ^ a[3] ^ b[1] ^ b[2]);
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(buf + o0[u]);
          acc += v.x ^ v.y ^ v.z ^ v.w;
        }
        asm volatile("" : "+v"(acc));
      }
    }
  }
  sink[static_cast<int64_t>(blockIdx.x) * 256 + t] = static_cast<float>(acc);
}

}  // namespace

void launch_probe_atomic(float* buf, int ntiles, int blocks, int iters, hipStream_t s) {
  timing_begin(kKProbeAtomic, s);
  hipLaunchKernelGGL(k_probe_atomic, dim3(blocks), dim3(256), 0, s, buf, ntiles, iters);
  timing_end(kKProbeAtomic, s);
}

void launch_probe_lds(float* sink, int blocks, int iters, int mode, hipStream_t s) {
  timing_begin(kKProbeLds, s);
  hipLaunchKernelGGL(k_probe_lds, dim3(blocks), dim3(256), 0, s, sink, iters, mode);
  timing_end(kKProbeLds, s);
}

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
