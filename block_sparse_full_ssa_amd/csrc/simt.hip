// Generic (SIMT) kernels of the two SSA attention streams.
//
// One wave per query row; each lane owns d/64 consecutive elements of the
// head dimension and every logit is a butterfly wave sum.  All arithmetic is
// fp32 with the accurate device expf/logf, so this path is the fp32 layer's
// implementation (exact-enough for 1e-5 parity) and serves every shape the
// bf16 MFMA kernels do not cover.  It streams keys in ascending order and
// advances through the row's ascending block list, so a key's block is
// either selected (sparse support: the key is visible to the sparse stream)
// or not, decided without any table.
//
// Forward (Sintesi Tecnica, section 2): one pass over keys 0..t updates the
// online-softmax state of the full stream always and of the sparse stream on
// selected keys; the epilogue writes h, lse, delta = 1 - exp(lse_s - lse_f)
// and the row's sum of (h_full - h_sparse)^2 for the alignment losses.
// Backward: per row, the stream gradients G_f / G_s (upstream gradient to the
// active stream, alignment gradients to both in dual modes), D = G . h, then
// per key dZ = p (G . v - D) feeds dq (in registers), and dk, dv through fp32
// atomics into zeroed accumulators.

#include <limits.h>

#include "common.h"
#include "internal.h"

namespace ssa {

template <typename T, int E>
__global__ void __launch_bounds__(256) k_fwd_simt(FwdArgs a, int Hq, int G, int N, int d, int block,
                                                  int K, float scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t bh = row / N;
  const int t = static_cast<int>(row % N);
  const int64_t bc = (bh / Hq) * (Hq / G) + (bh % Hq) / G;
  const bool want_full = a.mode != kSparseOnly;
  const bool want_sparse = a.mode != kFullOnly;

  const T* qp = static_cast<const T*>(a.q) + row * d + lane * E;
  const T* kp = static_cast<const T*>(a.k) + bc * N * d + lane * E;
  const T* vp = static_cast<const T*>(a.v) + bc * N * d + lane * E;
  const int32_t* selp = want_sparse ? a.sel + row * K : nullptr;

  float qv[E], of[E], os[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f32(qp[e]);
    of[e] = 0.f;
    os[e] = 0.f;
  }
  float mf = -INFINITY, lf = 0.f, ms = -INFINITY, ls = 0.f;
  // optional diagnostics: full-stream mass on the first key block, and
  // sum_i p_i (z_i - mf) with p_i = exp(z_i - mf), for the entropy
  const bool stats = want_full && a.sink_mass != nullptr;
  float sink_l = 0.f, ex_l = 0.f;
  int ptr = 0;
  // the row's entries in ascending order; negative entries are skipped, and
  // past the last entry no block matches
  int next_blk = want_sparse ? selp[0] : INT_MAX;

  for (int i = 0; i <= t; ++i) {
    float dot = 0.f;
    float vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      dot = fmaf(qv[e], to_f32(kp[static_cast<int64_t>(i) * d + e]), dot);
      vv[e] = to_f32(vp[static_cast<int64_t>(i) * d + e]);
    }
    const float z = wave_sum(dot) * scale;
    if (want_full) {
      const float mn = fmaxf(mf, z);
      const float al = expf(mf - mn), p = expf(z - mn);
      if (stats) {
        // a new maximum shifts every earlier exponent by mf - mn (al = 0 on the first key)
        ex_l = (al == 0.f ? 0.f : al * fmaf(mf - mn, lf, ex_l)) + p * (z - mn);
        sink_l = sink_l * al + (i < block ? p : 0.f);
      }
      lf = lf * al + p;
#pragma unroll
      for (int e = 0; e < E; ++e) of[e] = of[e] * al + p * vv[e];
      mf = mn;
    }
    if (want_sparse) {
      const int blk = i / block;
      while (next_blk < blk) {
        ++ptr;
        next_blk = ptr < K ? selp[ptr] : INT_MAX;
      }
      if (next_blk == blk) {
        const float mn = fmaxf(ms, z);
        const float al = expf(ms - mn), p = expf(z - mn);
        ls = ls * al + p;
#pragma unroll
        for (int e = 0; e < E; ++e) os[e] = os[e] * al + p * vv[e];
        ms = mn;
      }
    }
  }

  float sq = 0.f;
  const float inv_f = 1.f / lf, inv_s = 1.f / ls;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float hf = of[e] * inv_f, hs = os[e] * inv_s;
    if (want_full) static_cast<T*>(a.h_full)[row * d + lane * E + e] = from_f32<T>(hf);
    if (want_sparse) static_cast<T*>(a.h_sparse)[row * d + lane * E + e] = from_f32<T>(hs);
    if (want_full && want_sparse) sq += (hf - hs) * (hf - hs);
  }
  if (want_full && want_sparse) sq = wave_sum(sq);
  if (lane == 0) {
    const float lse_f = mf + logf(lf), lse_s = ms + logf(ls);
    if (want_full && a.lse_full) a.lse_full[row] = lse_f;
    if (want_sparse && a.lse_sparse) a.lse_sparse[row] = lse_s;
    if (want_full && want_sparse) {
      a.delta[row] = -expm1f(lse_s - lse_f);
      a.row_sq[row] = sq;
    }
    if (stats) {
      a.sink_mass[row] = sink_l / lf;
      a.entropy[row] = logf(lf) - ex_l / lf;
    }
  }
}

void launch_fwd_simt(const Dims& D, const FwdArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(D.rows() / 4));
  timing_begin(kKFwdSimt, s);
  if (D.dtype == 1) {
    if (D.d == 128)
      hipLaunchKernelGGL((k_fwd_simt<bf16_t, 2>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale);
    else
      hipLaunchKernelGGL((k_fwd_simt<bf16_t, 1>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale);
  } else {
    if (D.d == 128)
      hipLaunchKernelGGL((k_fwd_simt<float, 2>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale);
    else
      hipLaunchKernelGGL((k_fwd_simt<float, 1>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale);
  }
  timing_end(kKFwdSimt, s);
}

template <typename T, int E>
__global__ void __launch_bounds__(256) k_bwd_simt(BwdArgs a, int Hq, int G, int N, int d, int block,
                                                  int K, float scale, float inv_m) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t bh = row / N;
  const int t = static_cast<int>(row % N);
  const int64_t bc = (bh / Hq) * (Hq / G) + (bh % Hq) / G;
  const bool has_full = a.mode != kSparseOnly;
  const bool has_sparse = a.mode != kFullOnly;
  const bool dual = a.mode == kDualFull || a.mode == kDualSparse;
  const bool up_full = a.mode == kDualFull || a.mode == kFullOnly;

  const int64_t off = row * d + lane * E;
  const T* kp = static_cast<const T*>(a.k) + bc * N * d + lane * E;
  const T* vp = static_cast<const T*>(a.v) + bc * N * d + lane * E;
  float* dkp = a.dk_acc + bc * N * d + lane * E;
  float* dvp = a.dv_acc + bc * N * d + lane * E;
  const int32_t* selp = has_sparse ? a.sel + row * K : nullptr;

  float qv[E], gf[E], gs[E], dq[E];
  float Df = 0.f, Ds = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f32(static_cast<const T*>(a.q)[off + e]);
    const float g = a.dout ? to_f32(static_cast<const T*>(a.dout)[off + e]) : 0.f;
    const float hf = has_full ? to_f32(static_cast<const T*>(a.h_full)[off + e]) : 0.f;
    const float hs = has_sparse ? to_f32(static_cast<const T*>(a.h_sparse)[off + e]) : 0.f;
    if (dual) {
      const float diff = hf - hs;
      gf[e] = a.w_sparsity * 2.f * inv_m * diff + (up_full ? g : 0.f);
      gs[e] = -a.w_commit * 2.f * inv_m * diff + (up_full ? 0.f : g);
    } else {
      gf[e] = up_full ? g : 0.f;
      gs[e] = up_full ? 0.f : g;
    }
    Df += gf[e] * hf;
    Ds += gs[e] * hs;
    dq[e] = 0.f;
  }
  Df = wave_sum(Df);
  Ds = wave_sum(Ds);
  const float lse_f = has_full ? a.lse_full[row] : 0.f;
  const float lse_s = has_sparse ? a.lse_sparse[row] : 0.f;
  int ptr = 0;
  // the row's entries in ascending order; negative entries are skipped, and
  // past the last entry no block matches
  int next_blk = has_sparse ? selp[0] : INT_MAX;

  for (int i = 0; i <= t; ++i) {
    float kv[E], vv[E];
    float dot = 0.f, dpf = 0.f, dps = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kv[e] = to_f32(kp[static_cast<int64_t>(i) * d + e]);
      vv[e] = to_f32(vp[static_cast<int64_t>(i) * d + e]);
      dot = fmaf(qv[e], kv[e], dot);
      dpf = fmaf(gf[e], vv[e], dpf);
      dps = fmaf(gs[e], vv[e], dps);
    }
    const float z = wave_sum(dot) * scale;
    float ds = 0.f, pf = 0.f, ps = 0.f;
    if (has_full) {
      pf = expf(z - lse_f);
      ds += pf * (wave_sum(dpf) - Df);
    }
    if (has_sparse) {
      const int blk = i / block;
      while (next_blk < blk) {
        ++ptr;
        next_blk = ptr < K ? selp[ptr] : INT_MAX;
      }
      if (next_blk == blk) {
        ps = expf(z - lse_s);
        ds += ps * (wave_sum(dps) - Ds);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      dq[e] = fmaf(ds, kv[e], dq[e]);
      const float dkv = scale * ds * qv[e];
      const float dvv = pf * gf[e] + ps * gs[e];
      if (dkv != 0.f) atomicAdd(dkp + static_cast<int64_t>(i) * d + e, dkv);
      if (dvv != 0.f) atomicAdd(dvp + static_cast<int64_t>(i) * d + e, dvv);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) static_cast<T*>(a.dq)[off + e] = from_f32<T>(scale * dq[e]);
}

void launch_bwd_simt(const Dims& D, const BwdArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(D.rows() / 4));
  const float inv_m = static_cast<float>(1.0 / static_cast<double>(D.q_elems()));
  timing_begin(kKBwdSimt, s);
  if (D.dtype == 1) {
    if (D.d == 128)
      hipLaunchKernelGGL((k_bwd_simt<bf16_t, 2>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale, inv_m);
    else
      hipLaunchKernelGGL((k_bwd_simt<bf16_t, 1>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale, inv_m);
  } else {
    if (D.d == 128)
      hipLaunchKernelGGL((k_bwd_simt<float, 2>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale, inv_m);
    else
      hipLaunchKernelGGL((k_bwd_simt<float, 1>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.d, D.block, D.K, D.scale, inv_m);
  }
  timing_end(kKBwdSimt, s);
}

}  // namespace ssa
