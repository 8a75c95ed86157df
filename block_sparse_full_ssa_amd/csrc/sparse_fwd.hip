// Sparse-only forward of SSA on key-block buckets, bf16 MFMA on gfx950.
//
// The sparse stream alone (Sintesi Tecnica, section 2: softmax over the keys
// of each query's selected blocks, token-causal inside its own block) is
// computed key-block-stationary in two kernels:
//   part:  one workgroup per (batch, KV head, key block j) stages the
//          block's K and V in LDS and walks the bucket of rows that selected
//          j (all G query heads of the group) in batches of 32, one batch
//          per wave; each lane owns a row and loads the next batch's row
//          into registers while the current batch is written out.  Each row gets the block's
//          partial result: its softmax-normalised output over the block's
//          keys (bf16) and the block's log-sum-exp (fp32, log2 units),
//          stored at the row's bucket entry (a batch writes 32 consecutive
//          partials);
//   merge: per row, the partials of its selected blocks (found through the
//          bucket masks and word positions) are combined by their
//          log-sum-exps into h_sparse and lse_sparse.
// The matrix work is proportional to the selected (query, key) pairs; the
// partials make the pair HBM-bound (about 260 bytes written and read per
// selected (row, block)).
//
// Layout as in the fused forward: S^T = K Q^T (A = K rows from LDS, B = the
// gathered Q rows in registers) leaves lane l with query l % 32, and
// O^T += V^T P^T (V^T by LDS transpose reads) takes P^T straight from the
// S^T accumulator.  Nothing is copied HBM -> LDS asynchronously inside the
// loop, so the partial stores of one batch stay in flight during the next.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

// Physical 16-byte chunk of logical chunk c in a V row r (read by
// transposes), for head dimension HD (rows of 2 HD bytes): swz256 for
// 256-byte rows, swz128 for 128-byte rows.
template <int HD> __device__ __forceinline__ int swz_v(int r, int c) {
  return HD == 128 ? swz256(r, c) : swz128(r, c);
}

// Physical 16-byte chunk of logical chunk c in a K row r (read by rows).
template <int HD> __device__ __forceinline__ int swz_k(int r, int c) { return HD == 128 ? c ^ (r & 15) : swz128(r, c); }

template <int KH, int HD>   // the key block as KH halves of 32 keys; head dimension HD
__global__ void __launch_bounds__(256, (KH <= 2 ? 2 : 1)) k_sparse_part(SparseFwdArgs a, int Hq, int G, int N, int Nq,
                                                        int q_off, int nb, float scale_log2, int64_t spare) {
  constexpr int kBlk = 32 * KH;
  constexpr int kD = HD;
  constexpr int kCh = HD / 8;      // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlk * kD], Vs[kBlk * kD];
  // per-wave staging of a batch's partial outputs, so that they leave as
  // whole rows (4 consecutive partials of 256 bytes per store instruction)
  __shared__ __attribute__((aligned(16))) uint16_t Ot[4 * 32 * kD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, li = lane & 15;
  const int gk = grp >> 1, srow = li >> 2, m4 = li & 3;
  const int bc = blockIdx.x, j = blockIdx.y;
  const int Hkv = Hq / G;
  const int b = bc / Hkv, c = bc % Hkv;
  const int64_t bucket = static_cast<int64_t>(bc) * nb + j;
  const int p0 = a.offs[bucket];
  const int n = a.offs[bucket + 1] - p0;
  if (n == 0) return;
  const int32_t* list = a.rows + p0;
  const int64_t kvbase = (static_cast<int64_t>(bc) * N + static_cast<int64_t>(j) * kBlk) * kD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + kvbase;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + kvbase;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const int64_t qhead0 = static_cast<int64_t>(b) * Hq + c * G;   // first query head of the group

  // K and V blocks -> LDS, 16-byte chunks swizzled per row
  for (int e = tid; e < kBlk * kCh; e += 256) {
    const int r = e / kCh, cc = e % kCh;
    *reinterpret_cast<uint4*>(&Ks[r * kD + 8 * swz_k<HD>(r, cc)]) =
        *reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(r) * kD + 8 * cc);
    *reinterpret_cast<uint4*>(&Vs[r * kD + 8 * swz_v<HD>(r, cc)]) =
        *reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(r) * kD + 8 * cc);
  }
  __syncthreads();

  // The wave's batches are bt = wave, wave + 4, ...; lane col owns batch
  // row col (entry -1 past the bucket's end) and loads that row's Q as its
  // B operand: d = 16 ds + 8 g + s.
  // (Loads are unconditional, at a clamped index -- a lane past the
  // bucket's end takes its last entry, whose logits are then masked -- and
  // validity comes from the position alone: every batch issues the same
  // memory instructions and no loaded value is combined before its use, so
  // the compiler's waits are for the loads they need.)
  const int nbat = (n + 31) >> 5;
  auto entry = [&](int bt) -> int { return list[min(bt * 32 + col, n - 1)]; };
  auto load_q = [&](int e, bf16x8* qb) {
    const int hl = e / Nq;
    const int64_t R = (qhead0 + hl) * Nq + (e - hl * Nq);
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds)
      qb[ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qg + R * kD + 16 * ds + 8 * g));
  };

  bf16x8 qb[kD / 16];
  int bt = wave;
  if (bt >= nbat) return;
  int e = entry(bt), e_next = entry(bt + 4);
  load_q(e, qb);
  for (; bt < nbat; bt += 4) {
    const int e_after = entry(bt + 8);
    const bool valid = bt * 32 + col < n;
    const int t = valid ? q_off + e % Nq : 0;       // the row's position
    // S^T for the block's keys (A: key 32 kh + col, d = 16 ds + 8 g + s), log2 units
    f32x16 s[KH];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) s[kh] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds)
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const int r = kh * 32 + col;
        s[kh] = mfma32x32x16(lds_read8(&Ks[r * kD + 8 * swz_k<HD>(r, 2 * ds + g)]), qb[ds], s[kh]);
      }
    __builtin_amdgcn_sched_barrier(0);    // keep the phases' operand reads apart (register pressure)
    // the next batch's rows load while this one's softmax, P V and stores run
    if (bt + 4 < nbat) load_q(e_next, qb);
    // own block: keys <= t
    const bool diag = valid && t / kBlk == j;
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = j * kBlk + kh * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        float x = s[kh][i] * scale_log2;
        if (!valid || (diag && key > t)) x = -INFINITY;
        s[kh][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m = valid ? mx : 0.f;      // a valid row always has key j * block <= t
    float sum = 0.f;
    constexpr int kDT = HD / 32;     // 32-column output tiles
    f32x16 o[kDT];
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) o[dt] = f32x16{};
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kh][i] = fast_exp2(s[kh][i] - m);
      // O^T += V^T P^T; V^T for k-step st: lane (d = 32 dt + col, g) holds
      // keys 32 kh + 16 st + 8 (s / 4) + 4 g + s % 4 (transpose reads)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // P in bf16; the row sum adds exactly these rounded weights
        const bf16x8 pb = to_bf16x8_sum(s[kh][8 * st], s[kh][8 * st + 1], s[kh][8 * st + 2], s[kh][8 * st + 3],
                                        s[kh][8 * st + 4], s[kh][8 * st + 5], s[kh][8 * st + 6], s[kh][8 * st + 7],
                                        sum);
        const int r0 = kh * 32 + st * 16 + 4 * gk + srow, r1 = r0 + 8;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const int cc = 4 * dt + 2 * (grp & 1) + (m4 >> 1), ee = 4 * (m4 & 1);
          const bf16x8 va =
              lds_tr_pair(&Vs[r0 * kD + 8 * swz_v<HD>(r0, cc) + ee], &Vs[r1 * kD + 8 * swz_v<HD>(r1, cc) + ee]);
          o[dt] = mfma32x32x16(va, pb, o[dt]);
        }
      }
    }
    sum += __shfl_xor(sum, 32, 64);
    __builtin_amdgcn_sched_barrier(0);
    // partials of entries p0 + 32 bt + r (the bucket's rows are contiguous):
    // O^T / sum -> LDS row col (16-byte chunk 4 dt + i4 of d at physical
    // chunk (4 dt + i4) ^ (col % kCh)), then kCh lanes store each row
    {
      const float inv = valid ? 1.f / sum : 0.f;
      uint16_t* ot = Ot + wave * 32 * kD;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16& od = o[dt];
          *reinterpret_cast<uint2*>(&ot[col * kD + 8 * ((4 * dt + i4) ^ (col & (kCh - 1))) + 4 * g]) =
              make_uint2(pack_bf16x2(od[4 * i4] * inv, od[4 * i4 + 1] * inv),
                         pack_bf16x2(od[4 * i4 + 2] * inv, od[4 * i4 + 3] * inv));
        }
      // Rows past the bucket's end go to the spare entry (`spare`, past
      // every bucket's): unconditional stores keep every batch's memory
      // instructions the same, so that the wait for the next batch's rows
      // does not also wait for these stores.  (Both lanes of a row store the
      // same log-sum-exp.)
      const int64_t pr0 = static_cast<int64_t>(p0) + bt * 32;
      const int rows_here = min(32, n - bt * 32);
      constexpr int kRowsSt = 64 / kCh;            // rows per store instruction
#pragma unroll
      for (int i = 0; i < 32 / kRowsSt; ++i) {
        const int r = kRowsSt * i + lane / kCh, pc = lane % kCh;
        const uint4 u = *reinterpret_cast<const uint4*>(&ot[r * kD + 8 * pc]);
        const int64_t dst = r < rows_here ? pr0 + r : spare;
        *reinterpret_cast<uint4*>(a.part_o + dst * kD + 8 * (pc ^ (r & (kCh - 1)))) = u;
      }
      a.part_lse[valid ? pr0 + col : spare] = m + fast_log2(sum);
    }
    e = e_next;
    e_next = e_after;
  }
}

// LR = HD / 8 lanes per row (8 dims each), 256 / LR rows per workgroup.  The
// partial of (row, selected block j) is the row's entry in bucket (b, c, j).
// Up to 64 selected blocks, lane i of a row looks up slots i, i + LR, ... in
// parallel and the positions and weights are then broadcast within the LR
// lanes; wider rows (every block of a long sequence) take the serial loop.
template <int HD>
__global__ void __launch_bounds__(256) k_sparse_merge(SparseFwdArgs a, int64_t rows, int Hq, int G, int Nq,
                                                      int q_off, int block, int nb, int K, int Kc) {
  constexpr int kD = HD;
  constexpr int LR = HD / 8;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / LR) + (threadIdx.x / LR);
  const int li = threadIdx.x % LR;
  const bool live = row < rows;
  const int64_t rr = live ? row : 0;
  const int64_t bh = rr / Nq;
  const int t = static_cast<int>(rr - bh * Nq);     // query row (bucket masks are indexed by rows)
  const int b = static_cast<int>(bh / Hq), h = static_cast<int>(bh % Hq);
  const int Hkv = Hq / G, nqt = Nq / 32;
  const int64_t bc = static_cast<int64_t>(b) * Hkv + h / G;
  const int hl = h % G, qt = t >> 5;
  const uint32_t below = (1u << (t & 31)) - 1u;
  const int32_t* s = a.sel + rr * K;
  // Entries that name no causal block (negative, or above the row's own
  // block) and repeats of the previous entry are ignored: the buckets hold
  // no partial for them.
  const int own = (q_off + t) / block;
  auto entry = [&](int e) -> int {
    const int j = s[e];
    return (j >= 0 && j <= own && (e == 0 || s[e - 1] != j)) ? j : -1;
  };
  auto pos_of = [&](int j) -> int64_t {
    const int64_t w = ((bc * nb + j) * G + hl) * nqt + qt;
    return a.wpos[w] + __popc(a.mask[w] & below);
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](int64_t p, float wt) {
    const uint4 u = *reinterpret_cast<const uint4*>(a.part_o + (p * kD + 8 * li));
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      acc[2 * k2] += wt * __uint_as_float(wd[k2] << 16);
      acc[2 * k2 + 1] += wt * __uint_as_float(wd[k2] & 0xffff0000u);
    }
  };
  float m = -INFINITY, L = 0.f;
  if (Kc <= 64) {
    constexpr int kSlots = 64 / LR;     // lookups per lane
    int64_t p[kSlots];
    float x[kSlots];
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int e = LR * r + li;
      const int j = (live && e < Kc) ? entry(e) : -1;
      p[r] = j >= 0 ? pos_of(j) : 0;
      x[r] = j >= 0 ? a.part_lse[p[r]] : -INFINITY;
      m = fmaxf(m, x[r]);
    }
#pragma unroll
    for (int off = LR / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, LR));
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const float wt = x[r] == -INFINITY ? 0.f : fast_exp2(x[r] - m);
      L += wt;
      if (LR * r >= Kc) continue;      // uniform
      // every slot's partial loads at once (an absent slot loads entry 0, a
      // real address, and its contribution is selected away), then the sums
      uint4 u[LR];
      float wv[LR];
#pragma unroll
      for (int i = 0; i < LR; ++i) {
        wv[i] = __shfl(wt, i, LR);
        const uint32_t plo = __shfl(static_cast<uint32_t>(p[r]), i, LR);
        const uint32_t phi = __shfl(static_cast<uint32_t>(p[r] >> 32), i, LR);
        const int64_t pi = wv[i] != 0.f ? (static_cast<int64_t>(phi) << 32) | plo : 0;
        u[i] = *reinterpret_cast<const uint4*>(a.part_o + (pi * kD + 8 * li));
      }
#pragma unroll
      for (int i = 0; i < LR; ++i) {
        const uint32_t wd[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const float lo = __uint_as_float(wd[k2] << 16), hi = __uint_as_float(wd[k2] & 0xffff0000u);
          acc[2 * k2] += wv[i] != 0.f ? wv[i] * lo : 0.f;
          acc[2 * k2 + 1] += wv[i] != 0.f ? wv[i] * hi : 0.f;
        }
      }
    }
#pragma unroll
    for (int off = LR / 2; off >= 1; off >>= 1) L += __shfl_xor(L, off, LR);
  } else if (live) {
    for (int e = 0; e < Kc; ++e) {
      const int j = entry(e);
      if (j >= 0) m = fmaxf(m, a.part_lse[pos_of(j)]);
    }
    for (int e = 0; e < Kc; ++e) {
      const int j = entry(e);
      if (j < 0) continue;
      const int64_t p = pos_of(j);
      const float wt = fast_exp2(a.part_lse[p] - m);
      L += wt;
      add(p, wt);
    }
  }
  if (!live) return;
  const float inv = 1.f / L;
  uint4 o;
  o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  o.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  o.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.h_sparse) + row * kD + 8 * li) = o;
  if (li == 0 && a.lse_sparse) a.lse_sparse[row] = (m + fast_log2(L)) * kLn2;
}

}  // namespace

bool sparse_fwd_supported(const Dims& D) { return D.dtype == 1 && (D.d == 128 || D.d == 64); }

void launch_sparse_fwd(const Dims& D, const SparseFwdArgs& a, hipStream_t s) {
  const int Kc = D.K < D.nb ? D.K : D.nb;
  const float scale_log2 = D.scale * 1.4426950408889634f;
  dim3 grid(D.B * D.Hkv, D.nb);
  auto go = [&](auto hd_tag) {
    constexpr int HD = decltype(hd_tag)::value;
    timing_begin(kKSparsePart, s);
    if (D.block == 32)
      hipLaunchKernelGGL((k_sparse_part<1, HD>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.Nq, D.q_off, D.nb,
                         scale_log2, bucket_capacity(D));
    else if (D.block == 64)
      hipLaunchKernelGGL((k_sparse_part<2, HD>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.Nq, D.q_off, D.nb,
                         scale_log2, bucket_capacity(D));
    else
      hipLaunchKernelGGL((k_sparse_part<4, HD>), grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.Nq, D.q_off, D.nb,
                         scale_log2, bucket_capacity(D));
    timing_end(kKSparsePart, s);
    constexpr int kRowsWg = 256 / (HD / 8);
    timing_begin(kKSparseMerge, s);
    hipLaunchKernelGGL(k_sparse_merge<HD>, dim3(static_cast<unsigned>((D.rows() + kRowsWg - 1) / kRowsWg)),
                       dim3(256), 0, s, a, D.rows(), D.Hq, D.G, D.Nq, D.q_off, D.block, D.nb, D.K, Kc);
    timing_end(kKSparseMerge, s);
  };
  if (D.d == 64) go(std::integral_constant<int, 64>{});
  else go(std::integral_constant<int, 128>{});
}

}  // namespace ssa
