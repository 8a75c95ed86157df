// Block selection for SSA's sparse stream.
//
// The pages say only that the sparse stream is block-sparse attention whose
// inference operations match MoBA (Sintesi Tecnica, section 2 and section 4
// 'Efficienza').  The rule used here: query t of block i_t scores every
// earlier key block j by q_t . mean(k over block j) in fp32, keeps its own
// block, and takes the top_k - 1 best earlier blocks, the lower index winning
// a tie.  sel rows are written ascending, padded with -1.
//
// Two kernels:
//   block_mean: mean of each key block, fp32, [B*Hkv][nb][d];
//   select:     one workgroup per (head, up to 64 rows of one query block);
//               candidate scores are computed into LDS (fp32 matrix
//               instructions up to 1024 key blocks, else fp32 FMAs chunk by
//               chunk), then a wave ranks each row by a bitwise threshold
//               search (see below).

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {

template <typename T>
__global__ void __launch_bounds__(128) k_block_mean(const T* __restrict__ k, float* __restrict__ mu,
                                                    int N, int d, int block, int nb) {
  const int j = blockIdx.x;          // key block
  const int64_t bc = blockIdx.y;     // batch * Hkv + kv head
  const T* src = k + (bc * N + static_cast<int64_t>(j) * block) * d;
  const float inv = 1.0f / static_cast<float>(block);   // block is a power of two: exact
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int r = 0; r < block; ++r) acc += to_f32(src[static_cast<int64_t>(r) * d + c]);
    mu[(bc * nb + j) * d + c] = acc * inv;
  }
}

void launch_block_mean(const Dims& D, const void* k, float* mu, hipStream_t s) {
  dim3 grid(D.nb, D.B * D.Hkv);
  timing_begin(kKBlockMean, s);
  if (D.dtype == 1)
    hipLaunchKernelGGL(k_block_mean<bf16_t>, grid, dim3(128), 0, s,
                       static_cast<const bf16_t*>(k), mu, D.N, D.d, D.block, D.nb);
  else
    hipLaunchKernelGGL(k_block_mean<float>, grid, dim3(128), 0, s,
                       static_cast<const float*>(k), mu, D.N, D.d, D.block, D.nb);
  timing_end(kKBlockMean, s);
}

constexpr int kSelChunk = 64;     // candidate blocks scored per pass

// Ranking of R rows whose candidate scores sit in LDS (scores[r * nb + j],
// j < i): see the kernel comments.  Wave w ranks rows w*RW.. in steps of 4*RW.
template <int TM>
__device__ __forceinline__ void rank_rows(const float* scores, int32_t* out0, int R, int nb, int K, int i, int keep,
                                          int lane, int wave) {
  constexpr int RW = TM <= 8 ? 2 : 1;
  const int nt = (i + 63) >> 6;     // registers holding candidates of this block
  for (int r0 = wave * RW; r0 < R; r0 += 4 * RW) {
    uint32_t u[RW][TM];
#pragma unroll
    for (int w = 0; w < RW; ++w)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int j = 64 * t + lane;
        // + 0.0f turns -0 into +0, so the two zeros tie as the values do
        u[w][t] = (t < nt && j < i) ? ordered_bits(scores[(r0 + w) * nb + j] + 0.0f) : 0u;
      }
    // codes of absent candidates are 0, below every threshold tried (>= 1)
    uint32_t th[RW];
    bool done[RW];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      th[w] = 0u;
      done[w] = false;
    }
    // Once exactly `keep` candidates are >= the threshold, lower bits can only
    // raise it within the gap below the keep-th largest code: the set >= th
    // and hence the result no longer change, so the search stops (uniform:
    // counts come from ballots).
    for (int bit = 31; bit >= 0; --bit) {
      bool all = true;
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        if (done[w]) continue;
        const uint32_t c = th[w] | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int t = 0; t < TM; ++t) cnt += __popcll(__ballot(u[w][t] >= c));
        th[w] = cnt >= keep ? c : th[w];
        done[w] = cnt == keep;
        all = all && done[w];
      }
      if (all) break;
    }
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      int32_t* out = out0 + static_cast<int64_t>(r0 + w) * K;
      int need = keep;              // places left for codes equal to th
#pragma unroll
      for (int t = 0; t < TM; ++t) need -= __popcll(__ballot(u[w][t] > th[w]));
      int base = 0;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        {
          uint64_t eq = __ballot(u[w][t] == th[w]);
          if (__popcll(eq) > need) {    // keep only the `need` lowest lanes
            uint64_t take = 0;
            for (int n = 0; n < need; ++n) {
              const uint64_t low = eq & (~eq + 1);
              take |= low;
              eq ^= low;
            }
            eq = take;
          }
          need -= __popcll(eq);
          const uint64_t won = __ballot(u[w][t] > th[w]) | eq;
          if ((won >> lane) & 1) {
            const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(won >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(won), 0));
            out[base + below] = 64 * t + lane;
          }
          base += __popcll(won);
        }
      }
      for (int slot = keep + lane; slot < K; slot += 64) out[slot] = (slot == keep) ? i : -1;
    }
  }
}


// One workgroup (256 threads) per R rows of one query block (R divides the
// block and R x nb fp32 scores fit in 64 KiB); the rows share the candidate
// blocks j < i.
//  1. Scores: candidates stream through in chunks of 64; each thread computes
//     a tile of R/16 rows x 4 candidates (q . mu in fp32, sequential over the
//     head dimension) into the row's score line in LDS.
//  2. Ranking, in registers: lane l of a wave holds the scores of candidates
//     l, l + 64, ..., l + 64 (TM - 1) of a row as order-preserving unsigned
//     codes.  A 32-step bitwise search (one ballot and popcount per register
//     per step) finds the largest code c with at least top_k - 1 candidates
//     >= c: the (top_k - 1)-th largest score.  Every candidate above c is
//     kept, and candidates equal to c fill the remaining places lowest index
//     first.  Candidate order is (register, lane) = block order, so prefix
//     counts of the ballots place the winners ascending.
template <typename T, int TM>
__global__ void __launch_bounds__(256) k_select(const T* __restrict__ q, const float* __restrict__ mu_all,
                                                int32_t* __restrict__ sel, int Hq, int G, int Nq,
                                                int q_off, int d, int block, int nb, int K, int R) {
  // LDS: q rows [R][d + 4], candidate block means [64][d + 4], scores [R][nb]
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int dp = d + 4;
  float* qs = smem;
  float* mus = qs + R * dp;
  float* scores = mus + kSelChunk * dp;
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int t0 = blockIdx.x * R;    // R divides block (and q_off), so all rows share i
  const int i = (q_off + t0) / block;   // own block = number of candidates
  const int keep = min(K - 1, i);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const T* qrow0 = q + (static_cast<int64_t>(bh) * Nq + t0) * d;
  int32_t* out0 = sel + (static_cast<int64_t>(bh) * Nq + t0) * K;

  if (keep == i || keep == 0) {
    // nothing to rank: every earlier block (keep == i) or none (top_k == 1)
    for (int e = tid; e < R * K; e += blockDim.x) {
      const int slot = e % K;
      out0[e] = slot < keep ? slot : (slot == keep ? i : -1);
    }
    return;
  }

  for (int e = tid; e < R * d / 8; e += blockDim.x) {
    const int r = (e * 8) / d, c0 = (e * 8) % d;
#pragma unroll
    for (int u = 0; u < 8; ++u) qs[r * dp + c0 + u] = to_f32(qrow0[r * d + c0 + u]);
  }

  // ---- 1. scores
  const float* mu = mu_all + bc * nb * d;
  const int rpt = R >= 16 ? R >> 4 : 1;   // rows per scoring thread
  const int rg = tid >> 4, cg = tid & 15;
  for (int j0 = 0; j0 < i; j0 += kSelChunk) {
    const int nc = min(kSelChunk, i - j0);
    __syncthreads();                // q staged; previous chunk's means consumed
    for (int e = tid; e < kSelChunk * d / 4; e += blockDim.x) {
      const int cc = (e * 4) / d, dd = (e * 4) % d;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cc < nc) v = *reinterpret_cast<const float4*>(mu + static_cast<int64_t>(j0 + cc) * d + dd);
      *reinterpret_cast<float4*>(mus + cc * dp + dd) = v;
    }
    __syncthreads();
    if (rg * rpt < R) {
      float acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
      for (int dd = 0; dd < d; dd += 4) {
        float4 mv[4], qv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) mv[c] = *reinterpret_cast<const float4*>(mus + (4 * cg + c) * dp + dd);
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (a < rpt) qv[a] = *reinterpret_cast<const float4*>(qs + (rg * rpt + a) * dp + dd);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if (a < rpt) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc[a][c] = fmaf(qv[a].x, mv[c].x, acc[a][c]);
              acc[a][c] = fmaf(qv[a].y, mv[c].y, acc[a][c]);
              acc[a][c] = fmaf(qv[a].z, mv[c].z, acc[a][c]);
              acc[a][c] = fmaf(qv[a].w, mv[c].w, acc[a][c]);
            }
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a < rpt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (4 * cg + c < nc) scores[(rg * rpt + a) * nb + j0 + 4 * cg + c] = acc[a][c];
    }
  }
  __syncthreads();

  rank_rows<TM>(scores, out0, R, nb, K, i, keep, lane, wave);
}

// Scores by fp32 matrix instructions (v_mfma_f32_32x32x2_f32), for up to
// 1024 key blocks: one workgroup per R = 32 or 64 rows of one query block;
// wave w computes the 32 x 32 score tiles (row tile w / CT, candidate tile
// w % CT of each chunk of 32 CT candidates) with the rows' q (A operand:
// lane (row l % 32, half g) holds d = (D/2) g .. (D/2) g + D/2 - 1) and the
// candidates' block means (B operand, same split of d) in registers; the
// scores go to LDS and the rows are ranked as above.  Products and sums are
// fp32 (their order differs from a sequential dot product only by rounding).
template <typename T, int TM, int D>
__global__ void __launch_bounds__(256) k_select_mfma(const T* __restrict__ q, const float* __restrict__ mu_all,
                                                     int32_t* __restrict__ sel, int Hq, int G, int Nq,
                                                     int q_off, int block, int nb, int K, int R) {
  extern __shared__ __attribute__((aligned(16))) float scores[];   // [R][nb]
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int t0 = blockIdx.x * R;    // R divides block (and q_off), so all rows share i
  const int i = (q_off + t0) / block;   // own block = number of candidates
  const int keep = min(K - 1, i);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t* out0 = sel + (static_cast<int64_t>(bh) * Nq + t0) * K;
  if (keep == i || keep == 0) {
    for (int e = tid; e < R * K; e += blockDim.x) {
      const int slot = e % K;
      out0[e] = slot < keep ? slot : (slot == keep ? i : -1);
    }
    return;
  }
  const int RT = R / 32, CT = 4 / RT;
  const int rt = wave / CT, ct = wave % CT;
  const int g = lane >> 5, col = lane & 31;
  constexpr int H = D / 2;
  // A operand: row 32 rt + col, d = H g + k
  float qa[H];
  {
    const T* qr = q + (static_cast<int64_t>(bh) * Nq + t0 + 32 * rt + col) * D + H * g;
#pragma unroll
    for (int k8 = 0; k8 < H; k8 += 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qa[k8 + e] = to_f32(qr[k8 + e]);
    }
  }
  const float* mu = mu_all + bc * nb * D;
  for (int c0 = 0; c0 < i; c0 += 32 * CT) {
    const int tile0 = c0 + 32 * ct;
    if (tile0 >= i) continue;                       // uniform
    const int cand = tile0 + col;
    const float* mr = mu + static_cast<int64_t>(min(cand, nb - 1)) * D + H * g;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int k4 = 0; k4 < H; k4 += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(mr + k4);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4], m4.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 1], m4.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 2], m4.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 3], m4.w, acc, 0, 0, 0);
    }
    // lane (candidate col, g): register e is row 8 (e / 4) + 4 g + e % 4
    if (cand < i) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        scores[(32 * rt + 8 * (e >> 2) + 4 * g + (e & 3)) * nb + cand] = acc[e];
    }
  }
  __syncthreads();
  rank_rows<TM>(scores, out0, R, nb, K, i, keep, lane, wave);
}

// R rows per workgroup for the matrix-scored kernel (0: not applicable).
static int mfma_rows(const Dims& D) {
  if (D.block >= 64 && 64 * D.nb * 4 <= 64 * 1024) return 64;
  if (32 * D.nb * 4 <= 128 * 1024) return 32;
  return 0;
}

template <typename T, int TM, int DD>
static void launch_select_mfma(const Dims& D, int R, const void* q, const float* mu, int32_t* sel, hipStream_t s) {
  dim3 grid(D.Nq / R, D.B * D.Hq);
  const size_t lds = static_cast<size_t>(R) * D.nb * sizeof(float);
  static size_t granted = 0;     // above 64 KiB of LDS must be requested
  if (lds > granted) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select_mfma<T, TM, DD>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    granted = lds;
  }
  hipLaunchKernelGGL((k_select_mfma<T, TM, DD>), grid, dim3(256), lds, s, static_cast<const T*>(q), mu, sel, D.Hq,
                     D.G, D.Nq, D.q_off, D.block, D.nb, D.K, R);
}

template <typename T, int TM>
static void launch_select_mfma_d(const Dims& D, int R, const void* q, const float* mu, int32_t* sel, hipStream_t s) {
  if (D.d == 64) launch_select_mfma<T, TM, 64>(D, R, q, mu, sel, s);
  else launch_select_mfma<T, TM, 128>(D, R, q, mu, sel, s);
}

template <typename T, int TM>
static void launch_select_tm(const Dims& D, const void* q, const float* mu, int32_t* sel, hipStream_t s) {
  int R = D.block < 64 ? D.block : 64;
  while (R > 4 && static_cast<size_t>(R) * D.nb * sizeof(float) > 65536) R >>= 1;
  dim3 grid(D.Nq / R, D.B * D.Hq);
  const size_t lds =
      (static_cast<size_t>(R + kSelChunk) * (D.d + 4) + static_cast<size_t>(R) * D.nb) * sizeof(float);
  static size_t granted = 0;     // above 64 KiB of LDS must be requested
  if (lds > granted) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<T, TM>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    granted = lds;
  }
  hipLaunchKernelGGL((k_select<T, TM>), grid, dim3(256), lds, s, static_cast<const T*>(q), mu, sel, D.Hq, D.G,
                     D.Nq, D.q_off, D.d, D.block, D.nb, D.K, R);
}

// TM = registers per lane for a row's candidates: ceil(nb / 64), rounded up
// to a power of two (nb <= 4096).
template <typename T>
static void launch_select_t(const Dims& D, const void* q, const float* mu, int32_t* sel, hipStream_t s) {
  const int tm = (D.nb + 63) / 64;
  const int R = mfma_rows(D);
  if (R) {
    if (tm <= 1) launch_select_mfma_d<T, 1>(D, R, q, mu, sel, s);
    else if (tm <= 2) launch_select_mfma_d<T, 2>(D, R, q, mu, sel, s);
    else if (tm <= 4) launch_select_mfma_d<T, 4>(D, R, q, mu, sel, s);
    else if (tm <= 8) launch_select_mfma_d<T, 8>(D, R, q, mu, sel, s);
    else launch_select_mfma_d<T, 16>(D, R, q, mu, sel, s);
    return;
  }
  if (tm <= 1) launch_select_tm<T, 1>(D, q, mu, sel, s);
  else if (tm <= 2) launch_select_tm<T, 2>(D, q, mu, sel, s);
  else if (tm <= 4) launch_select_tm<T, 4>(D, q, mu, sel, s);
  else if (tm <= 8) launch_select_tm<T, 8>(D, q, mu, sel, s);
  else if (tm <= 16) launch_select_tm<T, 16>(D, q, mu, sel, s);
  else if (tm <= 32) launch_select_tm<T, 32>(D, q, mu, sel, s);
  else launch_select_tm<T, 64>(D, q, mu, sel, s);
}

void launch_select(const Dims& D, const void* q, const float* mu, int32_t* sel, hipStream_t s) {
  timing_begin(kKSelect, s);
  if (D.dtype == 1) launch_select_t<bf16_t>(D, q, mu, sel, s);
  else launch_select_t<float>(D, q, mu, sel, s);
  timing_end(kKSelect, s);
}

}  // namespace ssa
