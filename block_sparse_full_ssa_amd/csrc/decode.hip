// Single-token decode over a KV cache: the inference regime in which sparse
// attention runs alone (Sintesi Tecnica, section 4, 'Efficienza': at
// inference SSA performs the operations of MoBA).  A new token at position
// t (its key and value already in the cache) attends either to every cached
// key 0..t (the full stream) or to the keys of its selected blocks (the
// sparse stream): its own block up to t and the top_k - 1 earlier blocks
// with the largest q . mean(k over the block), the lower index winning a
// tie -- the same rule as the training layer, scored against block means
// kept in a cache next to K and V.
//
// Three kernels:
//   k_cache_means    mean of the keys of cached blocks [j0, j1) -> fp32 cache
//   k_decode_select  one workgroup per (sequence, query head): scores of the
//                    complete earlier blocks, a 32-step threshold search on
//                    order-preserving codes, winners compacted in block order
//   k_decode_attend  one wave per part (a selected block, or a chunk of
//                    consecutive blocks for the full stream): lane = key for
//                    the logits, lane = two columns of d for P V; a part's
//                    (o, max, sum) go to the workspace
//   k_decode_merge   per (sequence, query head): the parts combined by their
//                    maxima and sums -> h (input dtype) and lse (natural log)
// Decode is bound by HBM (each selected key and value is read once per
// query head); none of it is a dense contraction worth the matrix cores.

#include "common.h"
#include "internal.h"

namespace ssa {
namespace {

constexpr float kLog2eD = 1.4426950408889634f;

template <typename T>
__global__ void __launch_bounds__(256) k_cache_means(const T* __restrict__ k, float* __restrict__ mu, int L, int d,
                                                     int block, int nbmax, int j0) {
  // workgroup (kv head slot, block j0 + y); thread = one column of d
  const int64_t bc = blockIdx.x;
  const int j = j0 + static_cast<int>(blockIdx.y);
  const int col = threadIdx.x;
  if (col >= d) return;
  const T* src = k + (bc * L + static_cast<int64_t>(j) * block) * d + col;
  float s = 0.f;
  for (int i = 0; i < block; ++i) s += to_f32(src[static_cast<int64_t>(i) * d]);
  mu[(bc * nbmax + j) * d + col] = s / static_cast<float>(block);
}

// Block-wide exclusive prefix count of a per-thread flag over 256 threads in
// thread order; returns the count before this thread and sets *total.
__device__ __forceinline__ int block_scan_flag(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int before_in_wave = __popcll(bal & ((uint64_t(1) << lane) - 1));
  __syncthreads();
  if (lane == 0) wsum[w] = __popcll(bal);
  __syncthreads();
  int before = before_in_wave;
  for (int u = 0; u < w; ++u) before += wsum[u];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return before;
}

// Eight consecutive elements of a row as fp32 (16-byte loads for bf16).
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename T>
__global__ void __launch_bounds__(256) k_decode_select(const T* __restrict__ q, const float* __restrict__ mu,
                                                       const int32_t* __restrict__ pos, int32_t* __restrict__ sel,
                                                       int Hq, int G, int d, int block, int nbmax, int K) {
  __shared__ float qs[128];
  __shared__ uint32_t codes[4096];
  __shared__ int wsum[4];
  __shared__ int cnt_s;
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / Hq), h = static_cast<int>(bh % Hq);
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int tid = threadIdx.x;
  const int t = min(max(pos[b], 0), nbmax * block - 1);   // positions outside the cache are clamped
  const int it = t / block;                         // own block
  const int keep = min(K - 1, it);                  // earlier blocks to keep
  int32_t* out = sel + bh * K;
  if (keep == it) {                                 // every earlier block is kept
    for (int p = tid; p < K; p += 256) out[p] = p <= it ? p : -1;
    return;
  }
  if (keep == 0) {                                  // top_k 1: the own block alone
    for (int p = tid; p < K; p += 256) out[p] = p == 0 ? it : -1;
    return;
  }
  if (tid < d) qs[tid] = to_f32(q[bh * d + tid]);
  __syncthreads();
  const float* muc = mu + bc * nbmax * d;
  for (int j = tid; j < it; j += 256) {
    const float4* m4 = reinterpret_cast<const float4*>(muc + static_cast<int64_t>(j) * d);
    float s = 0.f;
    for (int e = 0; e < d / 4; ++e) {
      const float4 m = m4[e];
      s = fmaf(qs[4 * e], m.x, s);
      s = fmaf(qs[4 * e + 1], m.y, s);
      s = fmaf(qs[4 * e + 2], m.z, s);
      s = fmaf(qs[4 * e + 3], m.w, s);
    }
    codes[j] = ordered_bits(s);
  }
  __syncthreads();
  // the keep-th largest code: the largest c with #{codes >= c} >= keep
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int n = 0;
    for (int j = tid; j < it; j += 256) n += codes[j] >= cand ? 1 : 0;
    n = static_cast<int>(wave_sum(static_cast<float>(n)));
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    if ((tid & 63) == 0) atomicAdd(&cnt_s, n);
    __syncthreads();
    if (cnt_s >= keep) thr = cand;
    __syncthreads();
  }
  // winners: codes above the threshold, then the lowest-index codes equal to it
  int n_gt = 0;
  {
    int n = 0;
    for (int j = tid; j < it; j += 256) n += codes[j] > thr ? 1 : 0;
    n = static_cast<int>(wave_sum(static_cast<float>(n)));
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    if ((tid & 63) == 0) atomicAdd(&cnt_s, n);
    __syncthreads();
    n_gt = cnt_s;
  }
  const int need_eq = keep - n_gt;
  int written = 0, eq_seen = 0;
  for (int j0 = 0; j0 < it; j0 += 256) {
    const int j = j0 + tid;
    const uint32_t cj = j < it ? codes[j] : 0u;
    const bool eq = j < it && cj == thr;
    int eq_total;
    const int eq_before = block_scan_flag(eq, wsum, &eq_total);
    const bool win = j < it && (cj > thr || (eq && eq_seen + eq_before < need_eq));
    int win_total;
    const int win_before = block_scan_flag(win, wsum, &win_total);
    if (win) out[written + win_before] = j;
    written += win_total;
    eq_seen += eq_total;
  }
  if (tid == 0) out[keep] = it;
  for (int p = keep + 1 + tid; p < K; p += 256) out[p] = -1;
}

// Part p of row bh covers blocks [first, last] (sparse: one selected block;
// full: a chunk of consecutive blocks).  One wave per part, 4 per workgroup.
template <typename T, int E>
__global__ void __launch_bounds__(256) k_decode_attend(const T* __restrict__ q, const T* __restrict__ kc,
                                                       const T* __restrict__ vc, const int32_t* __restrict__ pos,
                                                       const int32_t* __restrict__ sel, float* __restrict__ part_o,
                                                       float* __restrict__ part_ml, int Hq, int G, int L, int block,
                                                       int K, int chunk, int n_parts, float scale_log2) {
  constexpr int d = 64 * E;
  __shared__ float qs[4][d];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t bh = blockIdx.x;
  const int p = static_cast<int>(blockIdx.y) * 4 + w;
  const int b = static_cast<int>(bh / Hq), h = static_cast<int>(bh % Hq);
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int t = min(max(pos[b], 0), L - 1);        // positions outside the cache are clamped
  if (p >= n_parts) return;
  int first, last;                                   // blocks of this part
  if (sel) {
    first = last = sel[bh * K + p];
  } else {
    first = p * chunk;
    last = min(first + chunk - 1, t / block);
  }
  float* po = part_o + (bh * n_parts + p) * d;
  float* pml = part_ml + (bh * n_parts + p) * 2;
  if (first < 0 || first > t / block) {             // no keys: an empty part
    for (int e = 0; e < E; ++e) po[lane * E + e] = 0.f;
    if (lane == 0) {
      pml[0] = -INFINITY;
      pml[1] = 0.f;
    }
    return;
  }
  for (int e = 0; e < E; ++e) qs[w][lane * E + e] = to_f32(q[bh * d + lane * E + e]);
  const T* kb = kc + bc * L * d;
  const T* vb = vc + bc * L * d;
  const int k_end = min(t + 1, (last + 1) * block);  // keys [first * block, k_end)
  float m = -INFINITY, l = 0.f, o[E];
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int k0 = first * block; k0 < k_end; k0 += 64) {
    const int key = k0 + lane;
    float s = -INFINITY;
    if (key < k_end) {
      const T* kr = kb + static_cast<int64_t>(key) * d;
      float acc = 0.f;
#pragma unroll 4
      for (int e0 = 0; e0 < d; e0 += 8) {
        float x[8];
        load8(kr + e0, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(qs[w][e0 + i], x[i], acc);
      }
      s = acc * scale_log2;
    }
    const float mx = wave_max(s);                    // finite: key k0 <= t is always present
    const float mn = fmaxf(m, mx);
    const float al = exp2f(m - mn);
    const float pv = key < k_end ? exp2f(s - mn) : 0.f;
    l = l * al + wave_sum(pv);
    for (int e = 0; e < E; ++e) o[e] *= al;
    m = mn;
    ps[w][lane] = pv;
    __builtin_amdgcn_wave_barrier();
    const int nk = min(64, k_end - k0);
#pragma unroll 8
    for (int i = 0; i < nk; ++i) {
      const float pi = ps[w][i];
      const T* vr = vb + static_cast<int64_t>(k0 + i) * d + lane * E;
      for (int e = 0; e < E; ++e) o[e] = fmaf(pi, to_f32(vr[e]), o[e]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  for (int e = 0; e < E; ++e) po[lane * E + e] = o[e];
  if (lane == 0) {
    pml[0] = m;                                      // log2 units
    pml[1] = l;
  }
}

template <typename T>
__global__ void __launch_bounds__(128) k_decode_merge(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, T* __restrict__ h,
                                                      float* __restrict__ lse, int d, int n_parts) {
  const int64_t bh = blockIdx.x;
  const int col = threadIdx.x;
  const float* pml = part_ml + bh * n_parts * 2;
  float M = -INFINITY;
  for (int p = 0; p < n_parts; ++p) M = fmaxf(M, pml[2 * p]);
  float L = 0.f, o = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float mp = pml[2 * p];
    if (mp == -INFINITY) continue;
    const float f = exp2f(mp - M);
    L = fmaf(pml[2 * p + 1], f, L);
    if (col < d) o = fmaf(part_o[(bh * n_parts + p) * d + col], f, o);
  }
  if (col < d) h[bh * d + col] = from_f32<T>(o / L);
  if (col == 0 && lse) lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

int decode_parts(const Dims& D, bool sparse) {
  return sparse ? D.K : (D.nb + kDecodeChunk - 1) / kDecodeChunk;
}

void launch_cache_means(const Dims& D, const void* k, float* mu, int j0, int j1, hipStream_t s) {
  if (j1 <= j0) return;
  dim3 grid(static_cast<unsigned>(D.B * D.Hkv), static_cast<unsigned>(j1 - j0));
  timing_begin(kKDecode, s);
  if (D.dtype == 1)
    hipLaunchKernelGGL(k_cache_means<bf16_t>, grid, dim3(128), 0, s, static_cast<const bf16_t*>(k), mu, D.N, D.d,
                       D.block, D.nb, j0);
  else
    hipLaunchKernelGGL(k_cache_means<float>, grid, dim3(128), 0, s, static_cast<const float*>(k), mu, D.N, D.d,
                       D.block, D.nb, j0);
  timing_end(kKDecode, s);
}

void launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t s) {
  const bool sparse = a.sel != nullptr;
  const int P = decode_parts(D, sparse);
  const int64_t rows = static_cast<int64_t>(D.B) * D.Hq;
  const float sl2 = D.scale * kLog2eD;
  timing_begin(kKDecode, s);
  if (D.dtype == 1) {
    const bf16_t* q = static_cast<const bf16_t*>(a.q);
    if (sparse)
      hipLaunchKernelGGL(k_decode_select<bf16_t>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, q, a.mu,
                         a.pos, a.sel, D.Hq, D.G, D.d, D.block, D.nb, D.K);
    const dim3 grid(static_cast<unsigned>(rows), static_cast<unsigned>((P + 3) / 4));
    if (D.d == 128)
      hipLaunchKernelGGL((k_decode_attend<bf16_t, 2>), grid, dim3(256), 0, s, q,
                         static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v), a.pos, a.sel, a.part_o,
                         a.part_ml, D.Hq, D.G, D.N, D.block, D.K, kDecodeChunk, P, sl2);
    else
      hipLaunchKernelGGL((k_decode_attend<bf16_t, 1>), grid, dim3(256), 0, s, q,
                         static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v), a.pos, a.sel, a.part_o,
                         a.part_ml, D.Hq, D.G, D.N, D.block, D.K, kDecodeChunk, P, sl2);
    hipLaunchKernelGGL(k_decode_merge<bf16_t>, dim3(static_cast<unsigned>(rows)), dim3(128), 0, s, a.part_o,
                       a.part_ml, static_cast<bf16_t*>(a.h), a.lse, D.d, P);
  } else {
    const float* q = static_cast<const float*>(a.q);
    if (sparse)
      hipLaunchKernelGGL(k_decode_select<float>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, q, a.mu,
                         a.pos, a.sel, D.Hq, D.G, D.d, D.block, D.nb, D.K);
    const dim3 grid(static_cast<unsigned>(rows), static_cast<unsigned>((P + 3) / 4));
    if (D.d == 128)
      hipLaunchKernelGGL((k_decode_attend<float, 2>), grid, dim3(256), 0, s, q, static_cast<const float*>(a.k),
                         static_cast<const float*>(a.v), a.pos, a.sel, a.part_o, a.part_ml, D.Hq, D.G, D.N,
                         D.block, D.K, kDecodeChunk, P, sl2);
    else
      hipLaunchKernelGGL((k_decode_attend<float, 1>), grid, dim3(256), 0, s, q, static_cast<const float*>(a.k),
                         static_cast<const float*>(a.v), a.pos, a.sel, a.part_o, a.part_ml, D.Hq, D.G, D.N,
                         D.block, D.K, kDecodeChunk, P, sl2);
    hipLaunchKernelGGL(k_decode_merge<float>, dim3(static_cast<unsigned>(rows)), dim3(128), 0, s, a.part_o,
                       a.part_ml, static_cast<float*>(a.h), a.lse, D.d, P);
  }
  timing_end(kKDecode, s);
}

}  // namespace ssa
