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
//   block_mean: mean of each key block, stored transposed (muT[bc][dim][j]) so
//               that lanes reading consecutive blocks read consecutive words;
//   select:     one workgroup per (head, R rows of one query block); scores
//               for all candidates land in LDS, then each wave ranks its rows
//               with repeated 64-bit wave-max reductions of (score, -index).

#include "common.h"
#include "internal.h"

namespace ssa {

template <typename T>
__global__ void __launch_bounds__(128) k_block_mean(const T* __restrict__ k, float* __restrict__ muT,
                                                    int N, int d, int block, int nb) {
  const int j = blockIdx.x;          // key block
  const int64_t bc = blockIdx.y;     // batch * Hkv + kv head
  const T* src = k + (bc * N + static_cast<int64_t>(j) * block) * d;
  const float inv = 1.0f / static_cast<float>(block);   // block is a power of two: exact
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int r = 0; r < block; ++r) acc += to_f32(src[static_cast<int64_t>(r) * d + c]);
    muT[(bc * d + c) * nb + j] = acc * inv;
  }
}

void launch_block_mean(const Dims& D, const void* k, float* muT, hipStream_t s) {
  dim3 grid(D.nb, D.B * D.Hkv);
  timing_begin(kKBlockMean, s);
  if (D.dtype == 1)
    hipLaunchKernelGGL(k_block_mean<bf16_t>, grid, dim3(128), 0, s,
                       static_cast<const bf16_t*>(k), muT, D.N, D.d, D.block, D.nb);
  else
    hipLaunchKernelGGL(k_block_mean<float>, grid, dim3(128), 0, s,
                       static_cast<const float*>(k), muT, D.N, D.d, D.block, D.nb);
  timing_end(kKBlockMean, s);
}

// Rows of one query block handled by a workgroup; the score buffer R x nb
// fp32 stays within 32 KiB of LDS.
static int select_rows_per_wg(const Dims& D) {
  int r = 16;
  while (r > 1 && static_cast<int64_t>(r) * D.nb * 4 > 32768) r >>= 1;
  return r;
}

template <typename T>
__global__ void __launch_bounds__(256) k_select(const T* __restrict__ q, const float* __restrict__ muT,
                                                int32_t* __restrict__ sel, int Hq, int G, int N,
                                                int d, int block, int nb, int K, int R) {
  extern __shared__ float smem[];
  float* qs = smem;                 // [R][d]
  float* scores = smem + R * d;     // [R][nb]
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int t0 = blockIdx.x * R;    // R divides block, so all rows share i
  const int i = t0 / block;         // own block = number of candidates
  const int keep = min(K - 1, i);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* qrow0 = q + (static_cast<int64_t>(bh) * N + t0) * d;
  int32_t* out0 = sel + (static_cast<int64_t>(bh) * N + t0) * K;

  if (keep == i) {
    // every earlier block is kept: 0, 1, ..., i, then padding
    for (int e = threadIdx.x; e < R * K; e += blockDim.x) {
      int slot = e % K;
      out0[e] = slot <= i ? slot : -1;
    }
    return;
  }

  for (int e = threadIdx.x; e < R * d; e += blockDim.x) qs[e] = to_f32(qrow0[e]);
  __syncthreads();

  // scores[r][j] = q_r . mu_j, sequential fp32 FMA over the head dimension
  const float* mu = muT + bc * d * nb;
  for (int j0 = 0; j0 < i; j0 += 64) {
    const int j = j0 + lane;
    if (j < i) {
      for (int r = wave; r < R; r += 4) {
        float acc = 0.f;
        const float* qr = qs + r * d;
        for (int c = 0; c < d; ++c) acc = fmaf(qr[c], mu[static_cast<int64_t>(c) * nb + j], acc);
        scores[r * nb + j] = acc;
      }
    }
  }
  __syncthreads();

  for (int r = wave; r < R; r += 4) {
    float* sc = scores + r * nb;
    // best candidate of this lane: largest score, then smallest index
    auto lane_best = [&]() -> uint64_t {
      uint64_t best = 0;
      for (int j = lane; j < i; j += 64) {
        float v = sc[j];
        if (v != -INFINITY) {
          uint64_t key = (static_cast<uint64_t>(ordered_bits(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(j));
          best = key > best ? key : best;
        }
      }
      return best;
    };
    uint64_t mine = lane_best();
    int chosen = 0x7fffffff;        // lane m holds the m-th winner
    for (int m = 0; m < keep; ++m) {
      uint64_t top = wave_max_u64(mine);
      int j = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(top));
      if (lane == m) chosen = j;
      if ((j & 63) == lane) {       // owner removes it and rescans
        sc[j] = -INFINITY;
        mine = lane_best();
      }
    }
    // ascending order: rank of each winner among the winners
    int rank = 0;
    for (int m = 0; m < keep; ++m) {
      int other = __shfl(chosen, m, 64);
      rank += (other < chosen) ? 1 : 0;
    }
    int32_t* out = out0 + static_cast<int64_t>(r) * K;
    if (lane < keep) out[rank] = chosen;
    for (int slot = keep + lane; slot < K; slot += 64) out[slot] = (slot == keep) ? i : -1;
  }
}

void launch_select(const Dims& D, const void* q, const float* muT, int32_t* sel, hipStream_t s) {
  const int R = select_rows_per_wg(D);
  dim3 grid(D.N / R, D.B * D.Hq);
  size_t lds = static_cast<size_t>(R) * (D.d + D.nb) * sizeof(float);
  timing_begin(kKSelect, s);
  if (D.dtype == 1)
    hipLaunchKernelGGL(k_select<bf16_t>, grid, dim3(256), lds, s, static_cast<const bf16_t*>(q), muT, sel,
                       D.Hq, D.G, D.N, D.d, D.block, D.nb, D.K, R);
  else
    hipLaunchKernelGGL(k_select<float>, grid, dim3(256), lds, s, static_cast<const float*>(q), muT, sel,
                       D.Hq, D.G, D.N, D.d, D.block, D.nb, D.K, R);
  timing_end(kKSelect, s);
}

}  // namespace ssa
