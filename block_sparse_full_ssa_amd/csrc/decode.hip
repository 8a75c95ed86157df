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
// Kernels:
//   k_cache_means    mean of the keys of cached blocks [j0, j1) -> fp32 cache
//   k_decode_scores  one thread per (KV head, complete earlier block): the
//                    order-preserving codes of q . mu_j (fp32) for the G
//                    query heads, spread over many workgroups so that the
//                    block means stream in at full width, each read once
//   k_decode_topk    per (sequence, query head): a radix-256 threshold
//                    search on the codes, winners compacted in block order
//   k_decode_attend  one wave per part: a selected block of one query head
//                    (sparse), or a chunk of consecutive blocks for all the
//                    query heads of a KV head (full: each key and value row
//                    is read once for the group); lane = key for the logits,
//                    lane = (key group, 8 columns) for P V; the part's
//                    (o, max, sum) go to the workspace
//   k_decode_merge   per (sequence, query head): the parts' maxima, then
//                    the parts combined by their weights -> h and lse
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

// Scores of the complete earlier blocks: four threads per (KV head, block),
// each with a quarter of d, combined by two shuffles; the block mean mu_j is
// read once for the G query heads of the KV head (in passes of up to 8
// heads); code = order-preserving bits of q . mu_j (fp32) for j < own block.
template <typename T>
__global__ void __launch_bounds__(256) k_decode_scores(const T* __restrict__ q, const float* __restrict__ mu,
                                                       const int32_t* __restrict__ pos, uint32_t* __restrict__ codes,
                                                       int Hq, int G, int d, int block, int nbmax) {
  __shared__ float4 qs[8][32];
  const int64_t bc = blockIdx.x;
  const int Hkv = Hq / G;
  const int b = static_cast<int>(bc / Hkv), c = static_cast<int>(bc % Hkv);
  const int t = min(max(pos[b], 0), nbmax * block - 1);
  const int it = t / block;
  const int quarter = threadIdx.x & 3;
  const int j = static_cast<int>(blockIdx.y) * 64 + (threadIdx.x >> 2);
  if (static_cast<int>(blockIdx.y) * 64 >= it) return;          // uniform: no candidate here
  const int nq = d / 16;                                         // float4s per quarter
  const float4* m4 = reinterpret_cast<const float4*>(mu + (bc * nbmax + min(j, it - 1)) * d) + quarter * nq;
  float4 mv[8];                                                  // the block mean's quarter, loaded first
#pragma unroll
  for (int e = 0; e < 8; ++e) mv[e] = e < nq ? m4[e] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g0 = 0; g0 < G; g0 += 8) {
    const int ng = min(8, G - g0);
    __syncthreads();                                             // qs of the previous pass consumed
    for (int e = threadIdx.x; e < ng * (d / 4); e += 256) {
      const int g = e / (d / 4), x = 4 * (e % (d / 4));
      const T* qr = q + (static_cast<int64_t>(b) * Hq + c * G + g0 + g) * d + x;
      qs[g][e % (d / 4)] = make_float4(to_f32(qr[0]), to_f32(qr[1]), to_f32(qr[2]), to_f32(qr[3]));
    }
    __syncthreads();
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= nq) break;
      const float4 m = mv[e];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float4 x = qs[g][quarter * nq + e];
        acc[g] = fmaf(x.x, m.x, acc[g]);
        acc[g] = fmaf(x.y, m.y, acc[g]);
        acc[g] = fmaf(x.z, m.z, acc[g]);
        acc[g] = fmaf(x.w, m.w, acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      acc[g] += __shfl_xor(acc[g], 1, 64);
      acc[g] += __shfl_xor(acc[g], 2, 64);
    }
    if (j < it && quarter == 0)
      for (int g = 0; g < ng; ++g)
        codes[(static_cast<int64_t>(b) * Hq + c * G + g0 + g) * nbmax + j] = ordered_bits(acc[g]);
  }
}

// Per (sequence, query head): the own block and the top_k - 1 largest codes,
// ties to the lower block, written ascending with -1 padding.  Thread tid
// holds codes tid + 256 r (r < 16: up to 4096 blocks) in registers; the
// threshold is found digit by digit (radix 256, four rounds).
__global__ void __launch_bounds__(256) k_decode_topk(const uint32_t* __restrict__ codes_g,
                                                     const int32_t* __restrict__ pos, int32_t* __restrict__ sel,
                                                     int Hq, int block, int nbmax, int K) {
  constexpr int R = 16;
  __shared__ int wsum[4];
  __shared__ int hist[256];
  __shared__ int pick[3];
  __shared__ int list[64];
  __shared__ int n_list;
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / Hq);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int nr = (it + 255) / 256;                  // uniform
  uint32_t c[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = tid + 256 * r;
    c[r] = (r < nr && j < it) ? codes_g[bh * nbmax + j] : 0u;
  }
  // the keep-th largest code, 8 bits per round: a histogram of the next
  // digit among the codes that match the digits fixed so far, then the digit
  // whose suffix count reaches the number still to find
  uint32_t prefix = 0, mask = 0;
  int remaining = keep;                             // codes still to take at or below the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nr && tid + 256 * r < it && (c[r] & mask) == prefix) atomicAdd(&hist[(c[r] >> shift) & 255u], 1);
    __syncthreads();
    // suffix sums S(v) = #{matching codes with digit >= v}, v = tid
    const int hv = hist[tid];
    int sv = hv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_down(sv, off, 64);
      if (lane + off < 64) sv += y;
    }
    if (lane == 0) wsum[w] = sv;                    // the wave's total
    __syncthreads();
    for (int u = w + 1; u < 4; ++u) sv += wsum[u];
    if (sv >= remaining && sv - hv < remaining) {   // exactly one digit
      pick[0] = static_cast<int>(prefix | (static_cast<uint32_t>(tid) << shift));
      pick[1] = remaining - (sv - hv);
      pick[2] = hv;                                 // last round: the codes equal to the threshold
    }
    __syncthreads();
    prefix = static_cast<uint32_t>(pick[0]);
    remaining = pick[1];
    mask |= 255u << shift;
    __syncthreads();                                // pick and wsum are reused next round
  }
  const uint32_t thr = prefix;
  const int n_gt = keep - remaining;                // codes above thr
  const int n_eq = pick[2];
  const int need_eq = keep - n_gt;
  if (need_eq == n_eq) {
    // no tie at the threshold to break: the winners are the codes >= thr
    // (keep <= 63 of them, top_k <= 64 here); gathered in any order, then
    // sorted ascending by one wave
    if (tid == 0) n_list = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nr && tid + 256 * r < it && c[r] >= thr) list[atomicAdd(&n_list, 1)] = tid + 256 * r;
    __syncthreads();
    if (w == 0) {
      int v = lane < keep ? list[lane] : 0x7fffffff;
#pragma unroll
      for (int k2 = 2; k2 <= 64; k2 <<= 1)
#pragma unroll
        for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
          const int other = __shfl_xor(v, j2, 64);
          const bool ascending = (lane & k2) == 0, lower = (lane & j2) == 0;
          v = (lower == ascending) ? min(v, other) : max(v, other);
        }
      if (lane < keep) out[lane] = v;
      if (lane == 0) out[keep] = it;
    }
    for (int p = keep + 1 + tid; p < K; p += 256) out[p] = -1;
    return;
  }
  int written = 0, eq_seen = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nr) break;                             // uniform
    const int j = tid + 256 * r;
    const bool eq = j < it && c[r] == thr;
    int eq_total;
    const int eq_before = block_scan_flag(eq, wsum, &eq_total);
    const bool win = j < it && (c[r] > thr || (eq && eq_seen + eq_before < need_eq));
    int win_total;
    const int win_before = block_scan_flag(win, wsum, &win_total);
    if (win) out[written + win_before] = j;
    written += win_total;
    eq_seen += eq_total;
  }
  if (tid == 0) out[keep] = it;
  for (int p = keep + 1 + tid; p < K; p += 256) out[p] = -1;
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

// One wave per part: NH query heads of one KV head over the keys of blocks
// [first, last] up to position t.  Logits: lane = key (its key row read once
// for all NH heads).  P V: lane = (key group, 8 columns), each V row read
// once for all NH heads; the key groups are combined at the end of the part.
// Sparse: NH = 1, a part is one selected block of one query head.  Full:
// NH = the group's heads, a part is a chunk of consecutive blocks.
template <typename T, int D, int NH>
__global__ void __launch_bounds__(256) k_decode_attend(const T* __restrict__ q, const T* __restrict__ kc,
                                                       const T* __restrict__ vc, const int32_t* __restrict__ pos,
                                                       const int32_t* __restrict__ sel, float* __restrict__ part_o,
                                                       float* __restrict__ part_ml, int Hq, int G, int L, int block,
                                                       int K, int chunk, int n_parts, float scale_log2) {
  constexpr int LPR = D / 8;          // lanes per row (8 columns each)
  constexpr int KG = 64 / LPR;        // key groups in P V
  __shared__ float4 qs[4][NH][D / 4];
  __shared__ float ps[4][NH][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t unit = blockIdx.x;    // NH = 1: a query row (b, h); NH = G: a KV head (b, c)
  const int p = static_cast<int>(blockIdx.y) * 4 + w;
  if (p >= n_parts) return;
  int b, h0;
  int64_t bc;
  if (NH == 1) {
    b = static_cast<int>(unit / Hq);
    h0 = static_cast<int>(unit % Hq);
    bc = static_cast<int64_t>(b) * (Hq / G) + h0 / G;
  } else {
    const int Hkv = Hq / G;
    b = static_cast<int>(unit / Hkv);
    bc = unit;
    h0 = static_cast<int>(unit % Hkv) * G;
  }
  const int t = min(max(pos[b], 0), L - 1);        // positions outside the cache are clamped
  int first, last;
  if (sel) {
    first = last = sel[unit * K + p];
  } else {
    first = p * chunk;
    last = min(first + chunk - 1, t / block);
  }
  const int64_t row0 = static_cast<int64_t>(b) * Hq + h0;   // output row of head h0
  if (first < 0 || first > t / block) {             // no keys: an empty part
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float* po = part_o + ((row0 + hh) * n_parts + p) * D;
      for (int e = lane; e < D; e += 64) po[e] = 0.f;
      if (lane == 0) {
        part_ml[((row0 + hh) * n_parts + p) * 2] = -INFINITY;
        part_ml[((row0 + hh) * n_parts + p) * 2 + 1] = 0.f;
      }
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
    if (lane < D / 4) {
      const T* qr = q + (row0 + hh) * D + 4 * lane;
      qs[w][hh][lane] = make_float4(to_f32(qr[0]), to_f32(qr[1]), to_f32(qr[2]), to_f32(qr[3]));
    }
  __builtin_amdgcn_wave_barrier();
  const T* kb = kc + bc * L * D;
  const T* vb = vc + bc * L * D;
  const int k_end = min(t + 1, (last + 1) * block);  // keys [first * block, k_end)
  const int kg = lane / LPR, cc = (lane % LPR) * 8;
  float m[NH], l[NH], o[NH][8];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  for (int k0 = first * block; k0 < k_end; k0 += 64) {
    const int key = k0 + lane;
    float s[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) s[hh] = -INFINITY;
    if (key < k_end) {
      const T* kr = kb + static_cast<int64_t>(key) * D;
      float acc[NH];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) acc[hh] = 0.f;
#pragma unroll
      for (int e0 = 0; e0 < D; e0 += 8) {
        float x[8];
        load8(kr + e0, x);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float4 a = qs[w][hh][e0 / 4], c = qs[w][hh][e0 / 4 + 1];
          acc[hh] = fmaf(a.x, x[0], acc[hh]);
          acc[hh] = fmaf(a.y, x[1], acc[hh]);
          acc[hh] = fmaf(a.z, x[2], acc[hh]);
          acc[hh] = fmaf(a.w, x[3], acc[hh]);
          acc[hh] = fmaf(c.x, x[4], acc[hh]);
          acc[hh] = fmaf(c.y, x[5], acc[hh]);
          acc[hh] = fmaf(c.z, x[6], acc[hh]);
          acc[hh] = fmaf(c.w, x[7], acc[hh]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) s[hh] = acc[hh] * scale_log2;
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const float mx = wave_max(s[hh]);              // finite: key k0 <= t is present
      const float mn = fmaxf(m[hh], mx);
      const float al = exp2f(m[hh] - mn);
      const float pv = key < k_end ? exp2f(s[hh] - mn) : 0.f;
      l[hh] = l[hh] * al + wave_sum(pv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= al;
      m[hh] = mn;
      ps[w][hh][lane] = pv;
    }
    __builtin_amdgcn_wave_barrier();
    const int nk = min(64, k_end - k0);
    if (nk == 64) {                                  // a whole group: every V load in flight at once
      float x[64 / KG][8];
#pragma unroll
      for (int j = 0; j < 64 / KG; ++j) load8(vb + static_cast<int64_t>(k0 + kg + KG * j) * D + cc, x[j]);
#pragma unroll
      for (int j = 0; j < 64 / KG; ++j)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float pi = ps[w][hh][kg + KG * j];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pi, x[j][e], o[hh][e]);
        }
    } else {
      for (int i = kg; i < nk; i += KG) {
        float x[8];
        load8(vb + static_cast<int64_t>(k0 + i) * D + cc, x);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float pi = ps[w][hh][i];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pi, x[e], o[hh][e]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // combine the key groups: lanes with the same columns are LPR apart
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int off = LPR; off < 64; off <<= 1) o[hh][e] += __shfl_xor(o[hh][e], off, 64);
  if (kg == 0) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float4* po = reinterpret_cast<float4*>(part_o + ((row0 + hh) * n_parts + p) * D + cc);
      po[0] = make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
      po[1] = make_float4(o[hh][4], o[hh][5], o[hh][6], o[hh][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      part_ml[((row0 + hh) * n_parts + p) * 2] = m[hh];        // log2 units
      part_ml[((row0 + hh) * n_parts + p) * 2 + 1] = l[hh];
    }
  }
}

// Per (sequence, query head): the parts' maxima reduced first, then every
// column adds its parts' outputs with known weights (independent loads).
template <typename T>
__global__ void __launch_bounds__(128) k_decode_merge(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, T* __restrict__ h,
                                                      float* __restrict__ lse, int d, int n_parts) {
  __shared__ float red[2];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const float* pml = part_ml + bh * n_parts * 2;
  float mx = -INFINITY;
  for (int p = tid; p < n_parts; p += 128) mx = fmaxf(mx, pml[2 * p]);
  mx = wave_max(mx);
  if (lane == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);            // finite: the own block is never empty
  const int col = tid < d ? tid : 0;
  const float* po = part_o + bh * n_parts * d + col;
  float L = 0.f, o = 0.f;
#pragma unroll 8
  for (int p = 0; p < n_parts; ++p) {
    const float g = exp2f(pml[2 * p] - M);           // 0 for an empty part (max -inf)
    L = fmaf(pml[2 * p + 1], g, L);
    o = fmaf(po[static_cast<int64_t>(p) * d], g, o);
  }
  if (tid < d) h[bh * d + tid] = from_f32<T>(o / L);
  if (tid == 0 && lse) lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
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

template <typename T, int D, int NH>
static void attend(const Dims& Dm, const DecodeArgs& a, int units, int P, float sl2, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(units), static_cast<unsigned>((P + 3) / 4));
  hipLaunchKernelGGL((k_decode_attend<T, D, NH>), grid, dim3(256), 0, s, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.pos, a.sel, a.part_o, a.part_ml,
                     Dm.Hq, Dm.G, Dm.N, Dm.block, Dm.K, kDecodeChunk, P, sl2);
}

template <typename T, int D>
static void attend_all(const Dims& Dm, const DecodeArgs& a, int P, float sl2, hipStream_t s) {
  const int rows = Dm.B * Dm.Hq, kv = Dm.B * Dm.Hkv;
  if (a.sel) {                      // sparse: every query head has its own blocks
    attend<T, D, 1>(Dm, a, rows, P, sl2, s);
    return;
  }
  switch (Dm.G) {                   // full: the group's heads share each key and value row read
    case 2: attend<T, D, 2>(Dm, a, kv, P, sl2, s); break;
    case 4: attend<T, D, 4>(Dm, a, kv, P, sl2, s); break;
    case 8: attend<T, D, 8>(Dm, a, kv, P, sl2, s); break;
    default: attend<T, D, 1>(Dm, a, rows, P, sl2, s); break;
  }
}

void launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t s) {
  const bool sparse = a.sel != nullptr;
  const int P = decode_parts(D, sparse);
  const unsigned rows = static_cast<unsigned>(D.B * D.Hq), kvs = static_cast<unsigned>(D.B * D.Hkv);
  const float sl2 = D.scale * kLog2eD;
  timing_begin(kKDecode, s);
  if (D.dtype == 1) {
    if (sparse) {
      hipLaunchKernelGGL(k_decode_scores<bf16_t>, dim3(kvs, static_cast<unsigned>((D.nb + 63) / 64)), dim3(256), 0,
                         s, static_cast<const bf16_t*>(a.q), a.mu, a.pos, a.codes, D.Hq, D.G, D.d, D.block, D.nb);
      hipLaunchKernelGGL(k_decode_topk, dim3(rows), dim3(256), 0, s, a.codes, a.pos, a.sel, D.Hq, D.block, D.nb, D.K);
    }
    if (D.d == 128) attend_all<bf16_t, 128>(D, a, P, sl2, s);
    else attend_all<bf16_t, 64>(D, a, P, sl2, s);
    hipLaunchKernelGGL(k_decode_merge<bf16_t>, dim3(rows), dim3(128), 0, s, a.part_o, a.part_ml,
                       static_cast<bf16_t*>(a.h), a.lse, D.d, P);
  } else {
    if (sparse) {
      hipLaunchKernelGGL(k_decode_scores<float>, dim3(kvs, static_cast<unsigned>((D.nb + 63) / 64)), dim3(256), 0,
                         s, static_cast<const float*>(a.q), a.mu, a.pos, a.codes, D.Hq, D.G, D.d, D.block, D.nb);
      hipLaunchKernelGGL(k_decode_topk, dim3(rows), dim3(256), 0, s, a.codes, a.pos, a.sel, D.Hq, D.block, D.nb, D.K);
    }
    if (D.d == 128) attend_all<float, 128>(D, a, P, sl2, s);
    else attend_all<float, 64>(D, a, P, sl2, s);
    hipLaunchKernelGGL(k_decode_merge<float>, dim3(rows), dim3(128), 0, s, a.part_o, a.part_ml,
                       static_cast<float*>(a.h), a.lse, D.d, P);
  }
  timing_end(kKDecode, s);
}

}  // namespace ssa
