// Block selection for SSA's sparse stream.
//
// The pages say only that the sparse stream is block-sparse attention whose
// inference operations match MoBA (Sintesi Tecnica, section 2 and section 4
// 'Efficienza').  The rule used here: query t of block i_t scores every
// earlier key block j by q_t . mean(k over block j) in fp32, keeps its own
// block, and takes the top_k - 1 best earlier blocks, the lower index winning
// a tie.  sel rows are written ascending, padded with -1.
//
// Kernels:
//   block_mean:  mean of each key block, fp32, [B*Hkv][nb][d];
//   split_means: (bf16 layers) each mean as the sum of two bf16 numbers;
//   select:      one workgroup per (head, 32 rows of one query block), the
//                row tiles of a KV head's query heads on one XCD, the
//                longest rows first; candidate scores are computed into LDS by matrix
//                instructions, up to 256 candidates at a time, and a wave
//                ranks each row by a bitwise threshold search (see below),
//                carrying a row's winners from one chunk of candidates into
//                the next.

#include <type_traits>

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

// Two-term bf16 split of the block means for bf16 layers: hi = bf16(mu),
// lo = bf16(mu - hi).  mu - hi is exact in fp32 and lo rounds it to 8 bits,
// so |mu - hi - lo| <= 2^-18 |mu|: the bf16 matrix products q.hi + q.lo
// (exact products, fp32 sums) give the fp32 score up to that error.
__global__ void __launch_bounds__(256) k_split_means(const float4* __restrict__ mu, uint2* __restrict__ hi,
                                                     uint2* __restrict__ lo, int64_t n4) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n4;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const float4 m = mu[e];
    const uint2 h = make_uint2(pack_bf16x2(m.x, m.y), pack_bf16x2(m.z, m.w));
    const float hx = __uint_as_float(h.x << 16), hy = __uint_as_float(h.x & 0xffff0000u);
    const float hz = __uint_as_float(h.y << 16), hw = __uint_as_float(h.y & 0xffff0000u);
    hi[e] = h;
    lo[e] = make_uint2(pack_bf16x2(m.x - hx, m.y - hy), pack_bf16x2(m.z - hz, m.w - hw));
  }
}

constexpr int kCand = 256;        // candidates scored and ranked per chunk
constexpr int kRows = 32;         // query rows per workgroup (divides every block size)
constexpr int kCarry = 64;        // carried winners per row (top_k <= 64 here)

// Ranking of R rows over one chunk of candidates (scores[r * CH + c] for the
// chunk's candidates c0 + c, c < nc) together with each row's winners so
// far (carried: codes and block indices, ascending, ncar of them), keeping
// `keep` winners.  Register slot 0 holds the carried entries (they precede
// every candidate of the chunk in block order), slots 1.. the chunk's
// candidates, so (slot, lane) order is block order: ties go to the lower
// block.  The winners replace the carried entries (ascending); on the last
// chunk they are written to the rows of sel instead, with the own block and
// the padding.  Without CARRY (every candidate in one chunk) there is no
// carried slot.  Wave w ranks rows w*RW.. in steps of 4*RW.
//
// After the first chunk (keep is then top_k - 1 throughout, as a chunk holds
// more candidates than that), a candidate whose code does not exceed the
// previous chunk's threshold car_th[r] cannot win: the carried entries are
// `keep` codes at or above it, and earlier blocks win ties.  The others are
// appended to the carried entries in LDS (block order kept); when they fit
// in one register slot the search runs over that slot alone.
template <int TM, bool CARRY>
__device__ __forceinline__ void rank_chunk(const float* scores, int CH, int c0, int nc, uint32_t* car_code,
                                           int32_t* car_idx, uint32_t* car_th, int ncar, int32_t* out0, int R,
                                           int K, int i, int keep, bool last, int lane, int wave) {
  constexpr int RW = 2;             // rows ranked together per wave
  constexpr int C0 = CARRY ? 1 : 0;  // first candidate slot
  constexpr int S = TM + C0;        // register slots: (carried +) candidates
  const int nt = (nc + 63) >> 6;    // candidate registers in use
  for (int r0 = wave * RW; r0 < R; r0 += 4 * RW) {
    uint32_t u[RW][S];
    int32_t cidx[RW];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      const int r = r0 + w;
      if (CARRY) {
        u[w][0] = lane < ncar ? car_code[r * kCarry + lane] : 0u;
        cidx[w] = lane < ncar ? car_idx[r * kCarry + lane] : 0;
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int c = 64 * t + lane;
        // + 0.0f turns -0 into +0, so the two zeros tie as the values do
        u[w][t + C0] = (t < nt && c < nc) ? ordered_bits(scores[r * CH + c] + 0.0f) : 0u;
      }
    }
    bool narrow = false;            // uniform: every live entry is in slot 0
    // start of the threshold search: bits above `bit0` of th are known
    uint32_t th0[RW];
    int bit0 = 31;
#pragma unroll
    for (int w = 0; w < RW; ++w) th0[w] = 0u;
    if constexpr (CARRY) {
      if (ncar > 0) {
        int live[RW];
        bool fit = true;
#pragma unroll
        for (int w = 0; w < RW; ++w) {
          const uint32_t th_old = car_th[r0 + w];
          int n = ncar;
#pragma unroll
          for (int t = C0; t < S; ++t) {
            u[w][t] = u[w][t] > th_old ? u[w][t] : 0u;
            n += __popcll(__ballot(u[w][t] != 0u));
          }
          live[w] = n;
          fit = fit && n <= 64;
        }
        if (fit) {
          narrow = true;
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const int r = r0 + w;
            int base = ncar;
#pragma unroll
            for (int t = C0; t < S; ++t) {
              const uint64_t b = __ballot(u[w][t] != 0u);
              if ((b >> lane) & 1) {
                const int pos = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0));
                car_code[r * kCarry + pos] = u[w][t];
                car_idx[r * kCarry + pos] = c0 + 64 * (t - C0) + lane;
              }
              base += __popcll(b);
            }
            // one wave owns the row: its LDS accesses complete in order
            u[w][0] = lane < live[w] ? car_code[r * kCarry + lane] : 0u;
            cidx[w] = lane < live[w] ? car_idx[r * kCarry + lane] : 0;
          }
          // The live codes lie between their minimum and maximum, so they
          // share the leading bits on which those two agree; the threshold
          // (between the keep-th largest code and the maximum) shares them
          // too, and the search starts below them.
          uint32_t mx[RW];
          int common = 32;
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const bool in = lane < live[w];
            mx[w] = wave_max_u32_dpp(in ? u[w][0] : 0u);
            const uint32_t mn = ~wave_max_u32_dpp(in ? ~u[w][0] : 0u);
            const int agree = (mx[w] ^ mn) == 0u ? 32 : __builtin_clz(mx[w] ^ mn);
            common = min(common, agree);
          }
          bit0 = 31 - common;
          const uint32_t top = common >= 32 ? 0xffffffffu : ~(0xffffffffu >> common);
#pragma unroll
          for (int w = 0; w < RW; ++w) th0[w] = mx[w] & top;
        }
      }
    }
    // threshold search and emission over the first NS register slots
    auto finish = [&](auto ns_tag) {
      constexpr int NS = decltype(ns_tag)::value;
      // codes of absent candidates are 0, below every threshold tried (>= 1)
      uint32_t th[RW];
      bool done[RW];
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        th[w] = th0[w];
        done[w] = false;
      }
      // Once exactly `keep` candidates are >= the threshold, lower bits can
      // only raise it within the gap below the keep-th largest code: the set
      // >= th and hence the result no longer change, so the search stops
      // (uniform: counts come from ballots).
      for (int bit = bit0; bit >= 0; --bit) {
        bool all = true;
#pragma unroll
        for (int w = 0; w < RW; ++w) {
          if (done[w]) continue;
          const uint32_t c = th[w] | (1u << bit);
          int cnt = 0;
#pragma unroll
          for (int t = 0; t < NS; ++t) cnt += __popcll(__ballot(u[w][t] >= c));
          th[w] = cnt >= keep ? c : th[w];
          done[w] = cnt == keep;
          all = all && done[w];
        }
        if (all) break;
      }
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        const int r = r0 + w;
        int32_t* out = out0 + static_cast<int64_t>(r) * K;
        int need = keep;              // places left for codes equal to th
#pragma unroll
        for (int t = 0; t < NS; ++t) need -= __popcll(__ballot(u[w][t] > th[w]));
        int base = 0;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
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
            const int idx = (CARRY && t == 0) ? cidx[w] : c0 + 64 * (t - C0) + lane;
            if (!CARRY || last) {
              out[base + below] = idx;
            } else {
              car_code[r * kCarry + base + below] = u[w][t];
              car_idx[r * kCarry + base + below] = idx;
            }
          }
          base += __popcll(won);
        }
        if (!CARRY || last) {
          for (int slot = keep + lane; slot < K; slot += 64) out[slot] = (slot == keep) ? i : -1;
        } else if (lane == 0) {
          car_th[r] = th[w];            // every winner's code is >= th
        }
      }
    };
    // only the slots that hold entries take part (uniform: nt is the chunk's)
    const int ns = C0 + nt;
    if (narrow || ns <= 1) finish(std::integral_constant<int, 1>{});
    else if (ns == 2) finish(std::integral_constant<int, (2 < S ? 2 : S)>{});
    else if (ns == 3) finish(std::integral_constant<int, (3 < S ? 3 : S)>{});
    else if (ns == 4) finish(std::integral_constant<int, (4 < S ? 4 : S)>{});
    else finish(std::integral_constant<int, S>{});
  }
}

// Scores by matrix instructions: one workgroup per R = 32 rows of one query
// block (R divides the block, so the rows share the candidate blocks j < i);
// wave w computes the 32 x 32 score tiles of candidate tile w of each pass
// over 128 candidates, with the rows' q as the A operand (in registers) and
// the candidates' block means as the B operand, into the rows' score lines
// in LDS.  bf16 layers: v_mfma_f32_32x32x16_bf16 on q (exact) and the two
// bf16 terms of each mean, into two accumulators added at the end (lane (row
// l % 32, half g) holds d = 16 s + 8 g .. +7 of step s).  fp32 layers:
// v_mfma_f32_32x32x2_f32 with lane (row l % 32, half g) holding d = (D/2) g
// .. (D/2) g + D/2 - 1.  Candidates go in chunks of
// up to 256: each chunk is scored, then ranked with the winners carried
// from the earlier chunks (rank_chunk).  Small chunks keep the LDS per
// workgroup at 48 KiB (three workgroups per CU) and the ranking's registers
// few; longer chunks measured slower at every length tried.  Products and
// sums are fp32 (their order differs from a sequential dot product only by
// rounding).
template <typename T, int TM, int D, bool CARRY>
__global__ void __launch_bounds__(256) k_select_mfma(const T* __restrict__ q, const float* __restrict__ mu_all,
                                                     const uint16_t* __restrict__ mu_hi,
                                                     const uint16_t* __restrict__ mu_lo, int32_t* __restrict__ sel,
                                                     int Hq, int G, int Nq, int q_off, int block, int nb, int K,
                                                     int R, int CH) {
  constexpr bool kBf = sizeof(T) == 2;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* scores = smem;                                                   // [R][CH]
  uint32_t* car_code = reinterpret_cast<uint32_t*>(smem + R * CH);       // [R][kCarry]
  int32_t* car_idx = reinterpret_cast<int32_t*>(car_code + R * kCarry);  // [R][kCarry]
  uint32_t* car_th = reinterpret_cast<uint32_t*>(car_idx + R * kCarry);  // [R]
  // work item: the row tiles of the G query heads of a KV head on one XCD
  // (its block means then stay in that XCD's L2), longest rows first
  const int n_rt = Nq / R;
  const QTileItem item = qtile_item(blockIdx.x, static_cast<int>(gridDim.x) / (n_rt * G), G, n_rt);
  const int bh = item.bh;
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const int t0 = (n_rt - 1 - item.rank) * R;    // R divides block (and q_off), so all rows share i
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
  // A operand of row 32 rt + col: bf16, d = 16 s + 8 g .. +7 in qb[s]; fp32,
  // d = H g + k in qa[k]
  float qa[kBf ? 1 : H];
  bf16x8 qb[kBf ? D / 16 : 1];
  {
    const T* qr = q + (static_cast<int64_t>(bh) * Nq + t0 + 32 * rt + col) * D;
    if constexpr (kBf) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qr + 16 * s + 8 * g));
    } else {
#pragma unroll
      for (int k = 0; k < H; ++k) qa[k] = to_f32(qr[H * g + k]);
    }
  }
  const float* mu = mu_all + bc * nb * D;
  auto score_chunk = [&](int c0, int nc) {
    for (int p0 = 0; p0 < nc; p0 += 32 * CT) {
      const int tile0 = p0 + 32 * ct;
      if (tile0 >= nc) continue;                    // uniform
      const int cand = c0 + tile0 + col;
      const int64_t mrow = (bc * nb + min(cand, nb - 1)) * D;
      f32x16 acc = f32x16{};
      if constexpr (kBf) {
        const uint16_t* mh = mu_hi + mrow + 8 * g;
        const uint16_t* ml = mu_lo + mrow + 8 * g;
        // the operands of half the k-steps in flight at once before their
        // products (interleaved with the products, the compiler keeps only
        // three loads in flight; all of them at once costs a wave per SIMD)
        f32x16 acc_lo = f32x16{};
        constexpr int kHalf = D / 32;       // k-steps per group of loads
#pragma unroll
        for (int s0 = 0; s0 < D / 16; s0 += kHalf) {
          bf16x8 bh[kHalf], bl[kHalf];
#pragma unroll
          for (int s = 0; s < kHalf; ++s) {
            bh[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(mh + 16 * (s0 + s)));
            bl[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ml + 16 * (s0 + s)));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < kHalf; ++s) {
            acc = mfma32x32x16(qb[s0 + s], bh[s], acc);
            acc_lo = mfma32x32x16(qb[s0 + s], bl[s], acc_lo);
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += acc_lo[e];
      } else {
        const float* mr = mu_all + mrow + H * g;
#pragma unroll
        for (int k4 = 0; k4 < H; k4 += 4) {
          const float4 m4 = *reinterpret_cast<const float4*>(mr + k4);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4], m4.x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 1], m4.y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 2], m4.z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[k4 + 3], m4.w, acc, 0, 0, 0);
        }
      }
      // lane (candidate col, g): register e is row 8 (e / 4) + 4 g + e % 4
      if (tile0 + col < nc) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          scores[(32 * rt + 8 * (e >> 2) + 4 * g + (e & 3)) * CH + tile0 + col] = acc[e];
      }
    }
    __syncthreads();
  };
  if constexpr (!CARRY) {
    // every candidate in one chunk: q is dead once the scores are in LDS
    score_chunk(0, i);
    rank_chunk<TM, false>(scores, CH, 0, i, car_code, car_idx, car_th, 0, out0, R, K, i, keep, true, lane, wave);
  } else {
    int ncar = 0;
    for (int c0 = 0; c0 < i; c0 += CH) {
      const int nc = min(CH, i - c0);
      if (c0 > 0) __syncthreads();                  // the previous chunk's scores consumed
      score_chunk(c0, nc);
      const bool last = c0 + CH >= i;
      const int keep_now = min(K - 1, c0 + nc);   // winners among the candidates so far
      rank_chunk<TM, true>(scores, CH, c0, nc, car_code, car_idx, car_th, ncar, out0, R, K, i, last ? keep : keep_now,
                           last, lane, wave);
      ncar = keep_now;
    }
  }
}

template <typename T, int TM, int DD, bool CARRY>
static void launch_select_mfma(const Dims& D, int R, const void* q, const float* mu, const uint16_t* mu_hi,
                               const uint16_t* mu_lo, int32_t* sel, hipStream_t s) {
  const int CH = D.nb < kCand ? D.nb : kCand;
  dim3 grid((D.Nq / R) * D.B * D.Hq);
  // the carried winners need LDS only when the candidates span several chunks
  // (at most 32 KiB of scores + 16 KiB of winners and their thresholds)
  const size_t lds = (static_cast<size_t>(R) * CH + (D.nb > CH ? (2 * static_cast<size_t>(kCarry) + 1) * R : 0)) *
                     sizeof(float);
  hipLaunchKernelGGL((k_select_mfma<T, TM, DD, CARRY>), grid, dim3(256), lds, s, static_cast<const T*>(q), mu, mu_hi,
                     mu_lo, sel, D.Hq, D.G, D.Nq, D.q_off, D.block, D.nb, D.K, R, CH);
}

template <typename T, int TM>
static void launch_select_mfma_d(const Dims& D, int R, const void* q, const float* mu, const uint16_t* mu_hi,
                                 const uint16_t* mu_lo, int32_t* sel, hipStream_t s) {
  const bool carry = D.nb > kCand;          // candidates in several chunks
  if (D.d == 64) {
    if (carry) launch_select_mfma<T, TM, 64, true>(D, R, q, mu, mu_hi, mu_lo, sel, s);
    else launch_select_mfma<T, TM, 64, false>(D, R, q, mu, mu_hi, mu_lo, sel, s);
  } else {
    if (carry) launch_select_mfma<T, TM, 128, true>(D, R, q, mu, mu_hi, mu_lo, sel, s);
    else launch_select_mfma<T, TM, 128, false>(D, R, q, mu, mu_hi, mu_lo, sel, s);
  }
}

// TM = registers per lane for a chunk's candidates: ceil(min(nb, 256) / 64),
// rounded up to a power of two.
template <typename T>
static void launch_select_t(const Dims& D, const void* q, const float* mu, const uint16_t* mu_hi,
                            const uint16_t* mu_lo, int32_t* sel, hipStream_t s) {
  const int tm = ((D.nb < kCand ? D.nb : kCand) + 63) / 64;
  if (tm <= 1) launch_select_mfma_d<T, 1>(D, kRows, q, mu, mu_hi, mu_lo, sel, s);
  else if (tm <= 2) launch_select_mfma_d<T, 2>(D, kRows, q, mu, mu_hi, mu_lo, sel, s);
  else launch_select_mfma_d<T, 4>(D, kRows, q, mu, mu_hi, mu_lo, sel, s);
}

size_t select_split_bytes(const Dims& D) {
  return D.dtype == 1 ? 2 * static_cast<size_t>(D.B) * D.Hkv * D.nb * D.d * sizeof(uint16_t) : 0;
}

void launch_select(const Dims& D, const void* q, const float* mu, uint16_t* split, int32_t* sel, hipStream_t s) {
  timing_begin(kKSelect, s);
  if (D.dtype == 1) {
    const int64_t n = static_cast<int64_t>(D.B) * D.Hkv * D.nb * D.d;   // d is a multiple of 4
    uint16_t* hi = split;
    uint16_t* lo = split + n;
    const int64_t n4 = n / 4;
    const int grid = static_cast<int>(n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096);
    hipLaunchKernelGGL(k_split_means, dim3(grid), dim3(256), 0, s, reinterpret_cast<const float4*>(mu),
                       reinterpret_cast<uint2*>(hi), reinterpret_cast<uint2*>(lo), n4);
    launch_select_t<bf16_t>(D, q, mu, hi, lo, sel, s);
  } else {
    launch_select_t<float>(D, q, mu, nullptr, nullptr, sel, s);
  }
  timing_end(kKSelect, s);
}

}  // namespace ssa
