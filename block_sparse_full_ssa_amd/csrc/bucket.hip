// Key-block buckets: the query rows that selected each key block.
//
// The sparse stream's support (Sintesi Tecnica, section 2: each query keeps
// its top-scoring key blocks plus its own block) is a per-row list of
// blocks.  The sparse-only kernels work key-block-stationary instead: for
// every (batch, KV head c, key block j) they need the rows of the G query
// heads of group c whose selection holds j, gathered into 32-row batches.
// Selections of neighbouring rows need not overlap, so a row-stationary
// tile would touch almost every key block; a bucket keeps the matrix work
// proportional to the selected pairs.
//
// Built in four steps, deterministic (no global atomics):
//   mask:  per (b, h, 32-row tile) of sel, one 32-bit row mask per key block
//          -> mask[b, c][j][h % G][tile]   (bit r: row 32 tile + r selected j),
//          a workgroup building the words of several consecutive tiles;
//   count: rows per bucket (popcounts of the bucket's masks);
//   scan:  exclusive prefix of the counts -> offs (one workgroup);
//   fill:  entries (h % G) * Nq + r of bucket (b, c, j) (r: the query row,
//          at position q_off + r), ordered by (head, r),
//          at rows[offs[(b*Hkv + c)*nb + j] ...], and for every mask word the
//          position of its first entry (wpos, same layout as mask), so that
//          the entry of (row, j) is wpos[word] + popcount of the word's bits
//          below the row.
// Entries of sel that are negative or above the row's own block are ignored.
// A layer has Nq = N query rows at positions 0 .. N-1 (q_off = 0); a prefill
// chunk has Nq rows at positions q_off .. (both multiples of 32 and of the
// block) against nb key blocks of the cache.

#include "common.h"
#include "internal.h"

namespace ssa {
namespace {

constexpr int kScanThreads = 256;

// Exclusive prefix sum over the 256 threads of a workgroup; *total receives
// the sum.  scratch: 4 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int x, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const int v = scratch[w];
    base += w < wave ? v : 0;
    sum += v;
  }
  __syncthreads();
  *total = sum;
  return base + incl - x;
}

// One workgroup per T consecutive 32-row tiles of one (b, h): the words of
// every key block for the T tiles are built in LDS and leave as runs of T
// consecutive words (the tiles of one block are adjacent in the layout).
// Words of blocks above a tile's own block are written as zeros; no reader
// looks at them.
__global__ void __launch_bounds__(kScanThreads) k_bucket_mask(const int32_t* __restrict__ sel,
                                                              uint32_t* __restrict__ mask, int Hq, int G, int Nq,
                                                              int q_off, int nb, int K, int block, int T) {
  extern __shared__ uint32_t words[];    // [own block of the last tile + 1][T]
  const int qt0 = blockIdx.x * T, bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int nqt = Nq / 32;
  const int nt = min(T, nqt - qt0);      // tiles of this workgroup
  const int b = bh / Hq, h = bh % Hq, Hkv = Hq / G;
  const int c = h / G, hl = h % G;
  const int own_last = (q_off + (qt0 + nt - 1) * 32) / block;   // block >= 32 divides into whole tiles
  const int nw = (own_last + 1) * T;
  for (int e = tid; e < nw; e += kScanThreads) words[e] = 0u;
  __syncthreads();
  for (int tt = 0; tt < nt; ++tt) {
    const int t0 = (qt0 + tt) * 32;
    const int own = (q_off + t0) / block;
    const int32_t* s = sel + (static_cast<int64_t>(bh) * Nq + t0) * K;
    for (int e = tid; e < 32 * K; e += kScanThreads) {
      const int blk = s[e];
      if (blk >= 0 && blk <= own) atomicOr(&words[blk * T + tt], 1u << (e / K));
    }
  }
  __syncthreads();
  uint32_t* out = mask + ((static_cast<int64_t>(b) * Hkv + c) * nb * G + hl) * nqt + qt0;
  for (int e = tid; e < nw; e += kScanThreads) {
    const int j = e / T, tt = e - j * T;
    if (tt < nt) out[static_cast<int64_t>(j) * G * nqt + tt] = words[e];
  }
}

__global__ void __launch_bounds__(kScanThreads) k_bucket_count(const uint32_t* __restrict__ mask,
                                                               int32_t* __restrict__ count, int G, int Nq,
                                                               int q_off, int nb, int block) {
  __shared__ int scratch[4];
  const int j = blockIdx.x, bc = blockIdx.y;
  const int nqt = Nq / 32;
  const int qt0 = max(0, j * block - q_off) / 32;   // earlier rows cannot select block j
  const uint32_t* m = mask + (static_cast<int64_t>(bc) * nb + j) * G * nqt;
  int cnt = 0;
  for (int hl = 0; hl < G; ++hl)
    for (int qt = qt0 + static_cast<int>(threadIdx.x); qt < nqt; qt += kScanThreads)
      cnt += __popc(m[static_cast<int64_t>(hl) * nqt + qt]);
  int total;
  block_exclusive_scan(cnt, scratch, &total);
  if (threadIdx.x == 0) count[static_cast<int64_t>(bc) * nb + j] = total;
}

// One workgroup: thread t sums its own contiguous run of counts, the runs'
// sums are scanned once, and each thread writes its run's offsets.
__global__ void __launch_bounds__(kScanThreads) k_bucket_scan(const int32_t* __restrict__ count,
                                                              int32_t* __restrict__ offs, int n) {
  __shared__ int scratch[4];
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int i0 = min(n, static_cast<int>(threadIdx.x) * per), i1 = min(n, i0 + per);
  int sum = 0;
  for (int i = i0; i < i1; ++i) sum += count[i];
  int total;
  int run = block_exclusive_scan(sum, scratch, &total);
  for (int i = i0; i < i1; ++i) {
    offs[i] = run;
    run += count[i];
  }
  if (threadIdx.x == 0) offs[n] = total;
}

__global__ void __launch_bounds__(kScanThreads) k_bucket_fill(const uint32_t* __restrict__ mask,
                                                              const int32_t* __restrict__ offs,
                                                              int32_t* __restrict__ rows,
                                                              int32_t* __restrict__ wpos, int G, int Nq,
                                                              int q_off, int nb, int block) {
  __shared__ int scratch[4];
  const int j = blockIdx.x, bc = blockIdx.y;
  const int nqt = Nq / 32;
  const int qt0 = max(0, j * block - q_off) / 32;
  const int64_t w0 = (static_cast<int64_t>(bc) * nb + j) * G * nqt;
  const uint32_t* m = mask + w0;
  int run = offs[static_cast<int64_t>(bc) * nb + j];
  for (int hl = 0; hl < G; ++hl) {
    for (int q0 = qt0; q0 < nqt; q0 += kScanThreads) {
      const int qt = q0 + static_cast<int>(threadIdx.x);
      uint32_t w = qt < nqt ? m[static_cast<int64_t>(hl) * nqt + qt] : 0u;
      int total;
      int pos = run + block_exclusive_scan(__popc(w), scratch, &total);
      if (qt < nqt) wpos[w0 + static_cast<int64_t>(hl) * nqt + qt] = pos;
      while (w) {
        const int r = __builtin_ctz(w);
        w &= w - 1;
        rows[pos++] = hl * Nq + 32 * qt + r;
      }
      run += total;
    }
  }
}

}  // namespace

int64_t bucket_mask_words(const Dims& D) {
  return static_cast<int64_t>(D.B) * D.Hkv * D.nb * D.G * (D.Nq / 32);
}

int64_t bucket_capacity(const Dims& D) {
  return D.rows() * static_cast<int64_t>(D.K < D.nb ? D.K : D.nb);
}

void launch_buckets(const Dims& D, const int32_t* sel, const Buckets& bk, hipStream_t s) {
  const int nbk = D.B * D.Hkv * D.nb;
  timing_begin(kKBucket, s);
  // tiles per mask workgroup: at most 32, and their words within 64 KiB of LDS
  int T = 1;
  while (T < 32 && static_cast<int64_t>(D.nb) * (2 * T) * 4 <= 65536) T *= 2;
  const int nqt = D.Nq / 32;
  hipLaunchKernelGGL(k_bucket_mask, dim3((nqt + T - 1) / T, D.B * D.Hq), dim3(kScanThreads),
                     static_cast<size_t>(D.nb) * T * 4, s, sel, bk.mask, D.Hq, D.G, D.Nq, D.q_off, D.nb, D.K,
                     D.block, T);
  hipLaunchKernelGGL(k_bucket_count, dim3(D.nb, D.B * D.Hkv), dim3(kScanThreads), 0, s, bk.mask, bk.count, D.G,
                     D.Nq, D.q_off, D.nb, D.block);
  hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(kScanThreads), 0, s, bk.count, bk.offs, nbk);
  hipLaunchKernelGGL(k_bucket_fill, dim3(D.nb, D.B * D.Hkv), dim3(kScanThreads), 0, s, bk.mask, bk.offs, bk.rows,
                     bk.wpos, D.G, D.Nq, D.q_off, D.nb, D.block);
  timing_end(kKBucket, s);
}

}  // namespace ssa
