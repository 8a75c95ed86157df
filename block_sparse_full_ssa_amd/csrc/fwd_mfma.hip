// Fused dual-stream forward of SSA attention, bf16 MFMA on gfx950.
//
// One pass over the causal key tiles feeds both streams of a training step
// (Sintesi Tecnica, section 2): the full stream (online softmax over every
// key <= t) and the sparse stream (online softmax over the keys of the
// query's selected blocks only, i.e. renormalised over that subset).  Both
// share the logits, so each K/V tile is staged in LDS once and S is computed
// once.  The epilogue writes both outputs, both log-sum-exps, the discarded
// mass delta(t) = 1 - exp(lse_sparse - lse_full) and each row's
// sum of (h_full - h_sparse)^2 for the alignment losses.
//
// Work split: a workgroup of 4 waves owns 128 consecutive queries of one
// head; each wave owns 32 of them.  Everything is kept transposed so that a
// lane owns one query:  S^T = K Q^T (A = K rows from LDS, B = the wave's Q in
// registers) leaves lane l with 16 keys of query l % 32 in its accumulator,
// the softmax statistics of a query live in one lane pair (l, l ^ 32), and
// O^T += V^T P^T (A = V^T via LDS transpose reads, B = P^T straight from the
// S^T accumulator) keeps the output of query l % 32 in lane l.  Keys are
// processed in halves of 32 so that the logits need 16 registers and both
// output accumulators stay in VGPRs.
//
// The head dimension HD (64 or 128) is a template parameter.  K/V tiles of
// 64 keys (32 for the full stream alone at HD = 128) move from HBM straight
// into LDS (buffer loads to LDS, 16 bytes per lane), double-buffered, one barrier
// per tile.  16-byte chunks are XOR-swizzled within each row so that
// the matrix-operand reads of K rows and the transpose reads of V columns
// avoid bank conflicts.
//
// Softmax: the running maxima are integers (ceil of a tile maximum) and move
// lazily, only when a tile exceeds them by more than kTau, so every rescale
// factor is an exact power of two (the full stream alone skips the tile
// maximum and moves its reference only when a tile's weights would pass
// 2^64).  In particular the sparse probabilities of
// a selected block are P_full * 2^(m_full - m_sparse), an exact fp32 product,
// whenever that exponent is at most 64; otherwise they are evaluated
// directly.  When every block is selected the two streams execute identical
// operations and agree bit for bit.  The probabilities enter the P V products
// in bf16 and the row sums add exactly those rounded values, so each output
// row is a weighted mean of value rows with the weights the products used.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kBM = 128;         // queries per workgroup
enum { kModeDual = 0, kModeFull = 1 };   // both streams / the full stream alone

// Keys per K/V tile and workgroups per CU, by head dimension D (128 or 64).
// D = 128: 64-key tiles for both streams (two workgroups per CU: both output
// accumulators take 128 registers), 32-key tiles for the full stream alone,
// whose smaller tiles (32 KiB of LDS) and registers (at most 168) let three
// workgroups share a CU.  D = 64 needs half the registers and LDS: 64-key
// tiles, three workgroups per CU with both streams and four with one.
template <int MODE, int D> struct FwdTile {
  static constexpr int kBN = (MODE == kModeFull && D == 128) ? 32 : 64;
  static constexpr int kTile = kBN * D;   // elements of one K or V tile
  static constexpr int kPerCu = D == 64 ? (MODE == kModeFull ? 4 : 3) : (MODE == kModeFull ? 3 : 2);
};
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTau = 8.f;      // lazy-rescale threshold (log2 units)



// Physical 16-byte chunk of logical chunk c in row r: K tiles are only read
// by rows, c ^ (r % 16) for 256-byte rows (D = 128); V tiles by transpose
// reads, swz256.  128-byte rows (D = 64): swz128 in both tiles.
template <int D> __device__ __forceinline__ int swz_k(int r, int c) {
  return D == 128 ? c ^ (r & 15) : swz128(r, c);
}
template <int D> __device__ __forceinline__ int swz_v(int r, int c) {
  return D == 128 ? swz256(r, c) : swz128(r, c);
}

__device__ __forceinline__ float max16(const f32x16& v) {
  // a chain of three-input maxima (v_max3_f32): two new values per instruction
  float m = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, v[i]), v[i + 1]);
  return __builtin_fmaxf(m, v[15]);
}

// Two to four workgroups per CU (see FwdTile), so one wave's softmax
// overlaps another wave's matrix work on every SIMD.
template <int MODE, bool STATS, int HD>
__global__ void __launch_bounds__(256, (FwdTile<MODE, HD>::kPerCu))
    k_fwd_mfma(FwdArgs a, int Hq, int G, int N, int Nq, int q_off, int block, int nb, int K, float scale_log2,
               int n_qtiles) {
  constexpr bool kSparse = MODE == kModeDual;
  // K and V tiles [kBN][HD] (swizzled), two of each; separate objects so that
  // the compiler can tell the tile being read from the one being filled
  constexpr int kBN = FwdTile<MODE, HD>::kBN;
  constexpr int kTile = FwdTile<MODE, HD>::kTile;
  __shared__ __attribute__((aligned(16))) uint16_t K0[kTile], K1[kTile], V0[kTile], V1[kTile];
  // dynamic LDS: the selection bits [kBM][W] of the rows
  extern __shared__ __attribute__((aligned(16))) uint32_t bits[];
  const int W = (nb + 31) >> 5;

  // The wave index and every condition that guards an MFMA are wave-uniform
  // for the compiler: matrix instructions must sit behind scalar branches,
  // never behind an EXEC mask.
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, li = lane & 15;
  const int gk = grp >> 1, srow = li >> 2, m4 = li & 3;
  const QTileItem item = qtile_item(blockIdx.x, static_cast<int>(gridDim.x) / (n_qtiles * G), G, n_qtiles);
  const int bh = item.bh;
  // positions: the query rows 0 .. Nq-1 sit at q_off .. qend-1 (a layer: q_off 0,
  // Nq = N); keys are the N positions of K / V
  const int q0 = q_off + (n_qtiles - 1 - item.rank) * kBM;   // longest tiles first
  const int qend = q_off + Nq;
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(bh) * Nq * HD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + bc * N * HD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + bc * N * HD;

  // ---- selection bits of the workgroup's rows
  if (kSparse) {
    for (int e = tid; e < kBM * W; e += 256) bits[e] = 0u;
    __syncthreads();
    for (int e = tid; e < kBM * K; e += 256) {
      const int r = e / K, t = q0 + r;
      if (t < qend) {
        const int blk = a.sel[(static_cast<int64_t>(bh) * Nq + (t - q_off)) * K + (e - r * K)];
        // entries outside 0 .. own block select nothing (and stay inside the row's words)
        if (blk >= 0 && blk <= t / block) atomicOr(&bits[r * W + (blk >> 5)], 1u << (blk & 31));
      }
    }
  }

  // ---- the wave's 32 queries as B operands (query = col, d = 16*ds + 8*g + s)
  const int qrow = q0 + wave * 32 + col;           // this lane's query
  const bool wave_live = q0 + wave * 32 < qend;
  const int wave_q0 = q0 + wave * 32;
  const int wave_last_q = min(qend - 1, wave_q0 + 31);
  bf16x8 qreg[HD / 16];
#pragma unroll
  for (int ds = 0; ds < HD / 16; ++ds) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < qend) u = *reinterpret_cast<const uint4*>(qg + static_cast<int64_t>(qrow - q_off) * HD + 16 * ds + 8 * g);
    qreg[ds] = __builtin_bit_cast(bf16x8, u);
  }

  constexpr int kDT = HD / 32;       // 32-column output tiles
  f32x16 of[kDT], os[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    of[dt] = f32x16{};
    os[dt] = f32x16{};
  }
  float mf = -INFINITY, lf = 0.f, ms = -INFINITY, ls = 0.f;
  // diagnostics (STATS): the full stream's mass on the first key block, and
  // sum_i e_i x_i with x_i = z_i log2(e) - mf and e_i = 2^x_i, both relative
  // to the running maximum like lf, for the entropy ln2 (log2 lf - ex / lf)
  float sink_l = 0.f, ex_l = 0.f, lfe = 0.f;   // lfe: the unrounded row sum (diagnostics)

  const int j_last = min(qend - 1, q0 + kBM - 1) / kBN;
  if (kSparse) __syncthreads();

  // HBM -> LDS copy of one K/V tile: each wave moves a quarter of its rows,
  // one 1 KiB instruction per kRowsOp rows; lane l fills physical chunk
  // l % (HD / 8) of row kRowsOp n + l / (HD / 8), so it fetches the logical chunk
  // stored there (byte offsets within the tile, fixed per lane).  Keys past the
  // end lie outside the tile's buffer resource and read zeros, which the causal
  // mask removes.
  constexpr int kRowsOp = 512 / HD;             // rows of one 1 KiB copy
  constexpr int kOps = kBN / kRowsOp / 4;      // copies per wave and tile
  uint32_t koff[kOps], voff[kOps];
#pragma unroll
  for (int r = 0; r < kOps; ++r) {
    const int row = kRowsOp * (wave * kOps + r) + lane / (HD / 8);
    const int p = lane % (HD / 8);
    koff[r] = 2 * (row * HD + 8 * swz_k<HD>(row, p));
    voff[r] = 2 * (row * HD + 8 * swz_v<HD>(row, p));
  }
  auto load_tile = [&](int j, uint16_t* Kd, uint16_t* Vd) {
    const int k0 = j * kBN;
    const uint32_t bytes = static_cast<uint32_t>(min(kBN, N - k0)) * (HD * 2);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg + static_cast<int64_t>(k0) * HD, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vg + static_cast<int64_t>(k0) * HD, bytes);
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      const int n = wave * kOps + r;
      buffer_to_lds16(rk, Kd + n * 512, koff[r]);
      buffer_to_lds16(rv, Vd + n * 512, voff[r]);
    }
  };

  // Byte offsets of the V transpose reads of rows 4 gk + srow and 8 further:
  // the swizzle term of those rows is 4 t + gk (+ 2), t = srow (HD = 128) or
  // (srow / 2) % 2 (HD = 64), so logical chunk 4 dt + y sits at physical
  // 4 (dt ^ t) + (y ^ gk (+ 2)); the term 32 t of the dt ^ t part is kept
  // apart on bits the rest leaves clear, so that column tile dt is an XOR of
  // 64 dt (bytes) and the row part (32 kh + 16 st2) a constant
  int tv[2];
  {
    const int y = 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
    const int t = HD == 128 ? srow : (srow >> 1) & 1;
    tv[0] = 2 * ((4 * gk + srow) * HD + 8 * (y ^ gk) + e4 + 32 * t);
    tv[1] = 2 * ((4 * gk + srow + 8) * HD + 8 * (y ^ (gk + 2)) + e4 + 32 * t);
  }

  // one tile: compute on (Ks, Vs) while the next streams into (Kn, Vn)
  auto step = [&](int j, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn) {
    if (j + 1 <= j_last) load_tile(j + 1, Kn, Vn);
  if (wave_live && j * kBN <= wave_last_q) {
#pragma unroll
    for (int kh = 0; kh < kBN / 32; ++kh) {
      const int kbase = j * kBN + kh * 32;          // first key of this half
      if (kbase > wave_last_q) break;               // uniform: later keys are all masked

      // selection bit of this half's key block for the lane's query
      bool sb = false;
      bool sparse_any = false;
      if (kSparse) {
        const int blk = kbase / block;
        sb = qrow < qend && blk < nb && ((bits[(wave * 32 + col) * W + (blk >> 5)] >> (blk & 31)) & 1u);
        sparse_any = __builtin_amdgcn_ballot_w64(sb) != 0;   // a scalar mask: uniform
      }

      // ---- S^T = K Q^T for 32 keys, in log2 units
      auto logits = [&]() {
        f32x16 acc = f32x16{};
        const int r = kh * 32 + col;
#pragma unroll
        for (int ds = 0; ds < HD / 16; ++ds)
          acc = mfma32x32x16(lds_read8(&Ks[r * HD + 8 * swz_k<HD>(r, 2 * ds + g)]), qreg[ds], acc);
        return acc;
      };
      f32x16 s = logits();
      // V^T operand of P V step u: key rows kh 32 + (u / kDT) 16 + 4 gk +
      // srow and 8 further (tv), column tile u % kDT; the row part is a
      // constant of the unrolled loops
      auto rd_vt = [&](int u) {
        const int x = 64 * (u % kDT), rb = 2 * HD * (kh * 32 + (u / kDT) * 16);
        return lds_tr_pair(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(Vs) + ((tv[0] ^ x) + rb)),
                           reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(Vs) + ((tv[1] ^ x) + rb)));
      };
      // (the diagnostics variant keeps its registers for its sums: no read-ahead)
      constexpr bool kAhead = !STATS;
      bf16x8 va_n, va_nn;
      if constexpr (kAhead) {
        va_n = rd_vt(0);
        va_nn = rd_vt(1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // logits stay unscaled: the scale (> 0) goes into the maximum and into
      // each exponent's fused multiply-add
      auto mask = [&](f32x16& x) {
        if (kbase + 31 > wave_q0) {                // uniform: the diagonal needs the causal mask
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > qrow) x[i] = -INFINITY;
          }
        }
      };
      mask(s);
      // The full stream alone keeps its reference maximum fixed and finds no
      // tile maximum: it takes the weights against the reference and moves
      // the reference (recomputing the tile's logits) only where a lane's
      // half-sum exceeds 2^64 or is not finite (a wave's first tile), so
      // every weight stays below 2^64 and every rescale is a power of two.
      constexpr bool kFixRef = MODE == kModeFull && !STATS;
      float mx = 0.f;
      if constexpr (!kFixRef) {
        mx = max16(s);
        mx = pair32_max(mx) * scale_log2;
      }

      // ---- new maxima (integers, moved lazily)
      float mfn = mf, alpha = 1.f;
      if constexpr (!kFixRef) {
        if (mx > mf + kTau) mfn = ceilf(mx);
        alpha = fast_exp2(mf - mfn);               // 1, 0 (first update) or an exact power of two
      }
      float msn = ms, alpha_s = 1.f;
      bool rescale = false;
      if (kSparse && sparse_any) {
        const float mxs = sb ? mx : -INFINITY;
        if (mxs > ms + kTau) msn = ceilf(mxs);
        alpha_s = msn == -INFINITY ? 1.f : fast_exp2(ms - msn);
        rescale = __builtin_amdgcn_ballot_w64(sb && mfn - msn > 64.f) == 0;
      }

      // ---- sparse probabilities evaluated directly (factor too large)
      bf16x8 ps[2];
      float sum_s = 0.f;
      if (kSparse && sparse_any && !rescale) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = sb ? fast_exp2(fmaf(s[8 * st + e], scale_log2, -msn)) : 0.f;
          ps[st] = to_bf16x8_sum(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], sum_s);
        }
      }

      // ---- full stream
      bf16x8 pf[2];
      float sum = 0.f, ex = 0.f, sume = 0.f;
      auto weights = [&]() {
        sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = fmaf(s[i], scale_log2, -mfn);
          if (STATS) x = fmaxf(x, -256.f);         // masked keys: e = 0 and e x = 0, not NaN
          s[i] = fast_exp2(x);
          if (STATS) {
            sume += s[i];
            ex = fmaf(s[i], x, ex);
          }
        }
        // P enters the products in bf16: round it here, and let the row sum
        // add exactly those weights
#pragma unroll
        for (int st = 0; st < 2; ++st)
          pf[st] = to_bf16x8_sum(s[8 * st], s[8 * st + 1], s[8 * st + 2], s[8 * st + 3], s[8 * st + 4],
                                 s[8 * st + 5], s[8 * st + 6], s[8 * st + 7], sum);
      };
      weights();
      if constexpr (kFixRef) {
        if (__builtin_amdgcn_ballot_w64(!(sum <= 0x1p64f)) != 0) {   // uniform, rare
          s = logits();
          mask(s);
          mx = pair32_max(max16(s)) * scale_log2;
          if (mx > mf + kTau) mfn = ceilf(mx);
          alpha = fast_exp2(mf - mfn);
          weights();
        }
      }
      if (STATS) {
        // the diagnostics use the unrounded weights: moving the maximum by
        // dm = mfn - mf shifts every earlier x by -dm and scales every earlier
        // e by alpha (0 on the first update)
        ex_l = (alpha == 0.f ? 0.f : alpha * fmaf(-(mfn - mf), lfe, ex_l)) + ex;
        sink_l = sink_l * alpha + (kbase < block ? sume : 0.f);
        lfe = lfe * alpha + sume;
      }
      lf = lf * alpha + sum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) of[dt] *= alpha;
      }
      mf = mfn;
      if (kSparse && sparse_any) {
        if (rescale) {
          // the factor c is a power of two, so each product s c is exact and
          // rounds to the full stream's rounded weight times c (c = 1 when
          // both maxima agree: then the weights and the sum are the full
          // stream's, bit for bit).  The lane's 16 keys lie in one block, so
          // its sparse half-sum is c times its full half-sum: scaling every
          // term of a rounded fp32 sum by a power of two scales the sum
          // exactly (weights below the bf16 normal range aside)
          const float c = sb ? fast_exp2(mfn - msn) : 0.f;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = s[8 * st + e] * c;
            ps[st] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          }
          sum_s = sum * c;
        }
        ls = ls * alpha_s + sum_s;
        if (__any(alpha_s != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) os[dt] *= alpha_s;
        }
        ms = msn;
      }

      // ---- O^T += V^T P^T over the 32 keys (two k-steps of 16); step u
      // is k-step u / kDT and column tile u % kDT, its V^T operand read two
      // steps ahead (the first two during the softmax)
#pragma unroll
      for (int u = 0; u < 2 * kDT; ++u) {
        bf16x8 va;
        if constexpr (kAhead) {
          va = va_n;
          va_n = va_nn;
          __builtin_amdgcn_sched_barrier(0);
          if (u + 2 < 2 * kDT) {
            va_nn = rd_vt(u + 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // the two reads before the products
          }
        } else {
          va = rd_vt(u);
        }
        of[u % kDT] = mfma32x32x16(va, pf[u / kDT], of[u % kDT]);
        if (kSparse && sparse_any) os[u % kDT] = mfma32x32x16(va, ps[u / kDT], os[u % kDT]);
      }
      if constexpr (kAhead) __builtin_amdgcn_sched_barrier(0);
    }
  }
    __builtin_amdgcn_s_waitcnt(0);     // the next tile has landed in LDS
    __syncthreads();
  };

  load_tile(0, K0, V0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j <= j_last; j += 2) {
    step(j, K0, V0, K1, V1);
    if (j + 1 > j_last) break;
    step(j + 1, K1, V1, K0, V0);
  }

  // ---- epilogue
  if (!wave_live) return;
  lf = pair32_sum(lf);
  if (STATS) {
    sink_l = pair32_sum(sink_l);
    ex_l = pair32_sum(ex_l);
    lfe = pair32_sum(lfe);
  }
  ls = pair32_sum(ls);
  const float inv_f = 1.f / lf, inv_s = 1.f / ls;
  const bool row_ok = qrow < qend;
  const int64_t row = static_cast<int64_t>(bh) * Nq + (qrow - q_off);
  float sq = 0.f;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dcol = 32 * dt + 8 * i4 + 4 * g;
      float hf[4], hs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hf[e] = of[dt][4 * i4 + e] * inv_f;
        hs[e] = os[dt][4 * i4 + e] * inv_s;
        if (MODE == kModeDual) sq += (hf[e] - hs[e]) * (hf[e] - hs[e]);
      }
      if (row_ok) {
        {
          uint2 u = make_uint2(pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h_full) + row * HD + dcol) = u;
        }
        if (kSparse) {
          uint2 u = make_uint2(pack_bf16x2(hs[0], hs[1]), pack_bf16x2(hs[2], hs[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h_sparse) + row * HD + dcol) = u;
        }
      }
    }
  }
  if (MODE == kModeDual) sq = pair32_sum(sq);
  if (row_ok && g == 0) {
    const float lse_f = (mf + fast_log2(lf)) * kLn2;
    const float lse_s = (ms + fast_log2(ls)) * kLn2;
    if (a.lse_full) a.lse_full[row] = lse_f;
    if (kSparse && a.lse_sparse) a.lse_sparse[row] = lse_s;
    if (MODE == kModeDual) {
      a.delta[row] = -expm1f(lse_s - lse_f);
      a.row_sq[row] = sq;
    }
    if (STATS) {
      a.sink_mass[row] = sink_l / lfe;
      a.entropy[row] = kLn2 * (fast_log2(lfe) - ex_l / lfe);
    }
  }
}

template <int MODE, bool STATS, int HD>
hipError_t launch_mode(const Dims& D, const FwdArgs& a, size_t lds, int n_qtiles, float scale_log2, hipStream_t s) {
  // LDS above 64 KiB in total must be granted per kernel; the grant is set on
  // every launch (the device current at the call), so no state is kept
  const void* fn = reinterpret_cast<const void*>(&k_fwd_mfma<MODE, STATS, HD>);
  if (lds > 0) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid(D.B * D.Hq * n_qtiles);   // work items from qtile_item
  hipLaunchKernelGGL((k_fwd_mfma<MODE, STATS, HD>), grid, dim3(256), lds, s, a, D.Hq, D.G, D.N, D.Nq, D.q_off, D.block,
                     D.nb, D.K, scale_log2, n_qtiles);
  return hipSuccess;
}

constexpr size_t kStaticLds = 4 * FwdTile<kModeDual, 128>::kTile * sizeof(uint16_t);   // the largest tiles

size_t lds_bytes(const Dims& D) {   // dynamic part: selection bits
  const int W = (D.nb + 31) / 32;
  return static_cast<size_t>(kBM * W) * sizeof(uint32_t);
}

}  // namespace

bool fwd_mfma_supported(const Dims& D) {
  // the selection bits of 128 rows must fit in LDS next to the K/V tiles
  return D.dtype == 1 && (D.d == 128 || D.d == 64) && kStaticLds + lds_bytes(D) <= 160 * 1024;
}

hipError_t launch_fwd_mfma(const Dims& D, const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (D.Nq + kBM - 1) / kBM;
  const size_t lds = a.mode == kFullOnly ? 0 : lds_bytes(D);   // the full stream reads no selection bits
  const float scale_log2 = D.scale * 1.4426950408889634f;
  timing_begin(kKFwdMfma, s);
  const bool stats = a.sink_mass != nullptr;
  hipError_t e;
  auto go = [&](auto d_tag) {
    constexpr int DD = decltype(d_tag)::value;
    if (a.mode == kFullOnly)
      return stats ? launch_mode<kModeFull, true, DD>(D, a, lds, n_qtiles, scale_log2, s)
                   : launch_mode<kModeFull, false, DD>(D, a, lds, n_qtiles, scale_log2, s);
    return stats ? launch_mode<kModeDual, true, DD>(D, a, lds, n_qtiles, scale_log2, s)
                 : launch_mode<kModeDual, false, DD>(D, a, lds, n_qtiles, scale_log2, s);
  };
  e = D.d == 64 ? go(std::integral_constant<int, 64>{}) : go(std::integral_constant<int, 128>{});
  timing_end(kKFwdMfma, s);
  return e;
}

}  // namespace ssa
