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
// K/V tiles of 64 keys move from HBM straight into LDS (global_load_lds,
// 16 bytes per lane), double-buffered, one barrier per tile.  16-byte chunks
// are XOR-swizzled within each 256-byte row so that the matrix-operand reads
// of K rows and the transpose reads of V columns avoid bank conflicts.
//
// Softmax: the running maxima are integers (ceil of a tile maximum) and move
// lazily, only when a tile exceeds them by more than kTau, so every rescale
// factor is an exact power of two.  In particular the sparse probabilities of
// a selected block are P_full * 2^(m_full - m_sparse), an exact fp32 product,
// whenever that exponent is at most 64; otherwise they are evaluated
// directly.  When every block is selected the two streams execute identical
// operations and agree bit for bit.

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kD = 128;          // head dimension
constexpr int kBM = 128;         // queries per workgroup
constexpr int kBN = 64;          // keys per tile
constexpr int kTile = kBN * kD;  // elements of one K or V tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTau = 8.f;      // lazy-rescale threshold (log2 units)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

enum { kModeDual = 0, kModeFull = 1 };   // both streams / the full stream alone

// Physical 16-byte chunk of logical chunk c in row r: K tiles are only read
// by rows; V tiles by transpose reads.
// The transposed tiles use c ^ (2 (r % 8) + (r / 8) % 2): measured on gfx950
// it keeps the transpose reads (ds_read_b64_tr_b16) free of bank conflicts
// as well as the 16-byte row reads, where c ^ (r % 8) or c ^ (r % 16) leave
// the transpose reads two-way conflicted.
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }

__device__ __forceinline__ float max16(const f32x16& v) {
  float m = fmaxf(v[0], v[1]);
#pragma unroll
  for (int i = 2; i < 16; i += 2) m = fmaxf(m, fmaxf(v[i], v[i + 1]));
  return m;
}

// Two workgroups per CU (256 VGPRs and 68 KiB of LDS each at nb <= 256), so
// one wave's softmax overlaps the other wave's matrix work on every SIMD.
template <int MODE, bool STATS>
__global__ void __launch_bounds__(256, 2)
    k_fwd_mfma(FwdArgs a, int Hq, int G, int N, int Nq, int q_off, int block, int nb, int K, float scale_log2,
               int n_qtiles) {
  constexpr bool kSparse = MODE == kModeDual;
  // K and V tiles [64][128] (swizzled), two of each; separate objects so that
  // the compiler can tell the tile being read from the one being filled
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
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(bh) * Nq * kD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + bc * N * kD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + bc * N * kD;

  // ---- selection bits of the workgroup's rows
  if (kSparse) {
    for (int e = tid; e < kBM * W; e += 256) bits[e] = 0u;
    __syncthreads();
    for (int e = tid; e < kBM * K; e += 256) {
      const int r = e / K, t = q0 + r;
      if (t < qend) {
        const int blk = a.sel[(static_cast<int64_t>(bh) * Nq + (t - q_off)) * K + (e - r * K)];
        if (blk >= 0) atomicOr(&bits[r * W + (blk >> 5)], 1u << (blk & 31));
      }
    }
  }

  // ---- the wave's 32 queries as B operands (query = col, d = 16*ds + 8*g + s)
  const int qrow = q0 + wave * 32 + col;           // this lane's query
  const bool wave_live = q0 + wave * 32 < qend;
  const int wave_q0 = q0 + wave * 32;
  const int wave_last_q = min(qend - 1, wave_q0 + 31);
  bf16x8 qreg[kD / 16];
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < qend) u = *reinterpret_cast<const uint4*>(qg + static_cast<int64_t>(qrow - q_off) * kD + 16 * ds + 8 * g);
    qreg[ds] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 of[4], os[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    of[dt] = f32x16{};
    os[dt] = f32x16{};
  }
  float mf = -INFINITY, lf = 0.f, ms = -INFINITY, ls = 0.f;
  // diagnostics (STATS): the full stream's mass on the first key block, and
  // sum_i e_i x_i with x_i = z_i log2(e) - mf and e_i = 2^x_i, both relative
  // to the running maximum like lf, for the entropy ln2 (log2 lf - ex / lf)
  float sink_l = 0.f, ex_l = 0.f;

  const int j_last = min(qend - 1, q0 + kBM - 1) / kBN;
  if (kSparse) __syncthreads();

  // HBM -> LDS copy of one K/V tile: each wave moves rows 16*wave .. +15, one
  // 1 KiB instruction per 4 rows; lane l fills physical chunk l % 16 of row
  // 4n + l / 16, so it fetches the logical chunk stored there.  Keys past the
  // end read the last key: finite values that the causal mask removes.
  auto load_tile = [&](int j, uint16_t* Kd, uint16_t* Vd) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = wave * 4 + r;
      const int row = 4 * n + (lane >> 4);
      const int p = lane & 15;
      const int64_t key = min(j * kBN + row, N - 1);
      const uint16_t* srck = kg + key * kD + 8 * swz_k(row, p);
      const uint16_t* srcv = vg + key * kD + 8 * swz_v(row, p);
      __builtin_amdgcn_global_load_lds((const glb_void*)srck, (lds_void*)(Kd + n * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const glb_void*)srcv, (lds_void*)(Vd + n * 512), 16, 0, 0);
    }
  };

  // one tile: compute on (Ks, Vs) while the next streams into (Kn, Vn)
  auto step = [&](int j, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn) {
    if (j + 1 <= j_last) load_tile(j + 1, Kn, Vn);
  if (wave_live && j * kBN <= wave_last_q) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kbase = j * kBN + kh * 32;          // first key of this half
      if (kbase > wave_last_q) break;               // uniform: later keys are all masked

      // selection bit of this half's key block for the lane's query
      bool sb = false;
      bool sparse_any = false;
      if (kSparse) {
        const int blk = kbase / block;
        sb = qrow < qend && blk < nb && ((bits[(wave * 32 + col) * W + (blk >> 5)] >> (blk & 31)) & 1u);
        sparse_any = __builtin_amdgcn_readfirstlane(__any(sb) ? 1 : 0) != 0;
      }

      // ---- S^T = K Q^T for 32 keys, in log2 units
      f32x16 s = f32x16{};
      {
        const int r = kh * 32 + col;
#pragma unroll
        for (int ds = 0; ds < kD / 16; ++ds)
          s = mfma32x32x16(lds_read8(&Ks[r * kD + 8 * swz_k(r, 2 * ds + g)]), qreg[ds], s);
      }
      // logits stay unscaled: the scale (> 0) goes into the maximum and into
      // each exponent's fused multiply-add
      if (kbase + 31 > wave_q0) {                  // uniform: the diagonal needs the causal mask
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key > qrow) s[i] = -INFINITY;
        }
      }
      float mx = max16(s);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;

      // ---- new maxima (integers, moved lazily)
      float mfn = mf, alpha = 1.f;
      if (mx > mf + kTau) mfn = ceilf(mx);
      alpha = fast_exp2(mf - mfn);                 // 1, 0 (first update) or an exact power of two
      float msn = ms, alpha_s = 1.f;
      bool rescale = false;
      if (kSparse && sparse_any) {
        const float mxs = sb ? mx : -INFINITY;
        if (mxs > ms + kTau) msn = ceilf(mxs);
        alpha_s = msn == -INFINITY ? 1.f : fast_exp2(ms - msn);
        rescale = __builtin_amdgcn_readfirstlane(__any(sb && mfn - msn > 64.f) ? 1 : 0) == 0;
      }

      // ---- sparse probabilities evaluated directly (factor too large)
      bf16x8 ps[2];
      float sum_s = 0.f;
      if (kSparse && sparse_any && !rescale) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = sb ? fast_exp2(fmaf(s[8 * st + e], scale_log2, -msn)) : 0.f;
            sum_s += p[e];
          }
          ps[st] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        }
      }

      // ---- full stream
      bf16x8 pf[2];
      float sum = 0.f, ex = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = fmaf(s[i], scale_log2, -mfn);
        if (STATS) x = fmaxf(x, -256.f);           // masked keys: e = 0 and e x = 0, not NaN
        s[i] = fast_exp2(x);
        sum += s[i];
        if (STATS) ex = fmaf(s[i], x, ex);
      }
      if (STATS) {
        // moving the maximum by dm = mfn - mf shifts every earlier x by -dm
        // and scales every earlier e by alpha (0 on the first update)
        ex_l = (alpha == 0.f ? 0.f : alpha * fmaf(-(mfn - mf), lf, ex_l)) + ex;
        sink_l = sink_l * alpha + (kbase < block ? sum : 0.f);
      }
      lf = lf * alpha + sum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) of[dt] *= alpha;
      }
      mf = mfn;
#pragma unroll
      for (int st = 0; st < 2; ++st)
        pf[st] = to_bf16x8(s[8 * st], s[8 * st + 1], s[8 * st + 2], s[8 * st + 3], s[8 * st + 4],
                           s[8 * st + 5], s[8 * st + 6], s[8 * st + 7]);
      if (kSparse && sparse_any) {
        if (rescale) {
          // exact: the factor is a power of two, so the row sum is the full
          // stream's sum of this half times it, bit for bit
          const float c = sb ? fast_exp2(mfn - msn) : 0.f;
          sum_s = sum * c;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = s[8 * st + e] * c;
            ps[st] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          }
        }
        ls = ls * alpha_s + sum_s;
        if (__any(alpha_s != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) os[dt] *= alpha_s;
        }
        ms = msn;
      }

      // ---- O^T += V^T P^T over the 32 keys (two k-steps of 16)
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2) {
        const int r0 = kh * 32 + st2 * 16 + 4 * gk + srow;   // key row of this lane's first read
        const int r1 = r0 + 8;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int c = 4 * dt + 2 * (grp & 1) + (m4 >> 1);   // logical 16-byte chunk
          const int e = 4 * (m4 & 1);
          const bf16x8 va = lds_tr_pair(&Vs[r0 * kD + 8 * swz_v(r0, c) + e], &Vs[r1 * kD + 8 * swz_v(r1, c) + e]);
          of[dt] = mfma32x32x16(va, pf[st2], of[dt]);
          if (kSparse && sparse_any) os[dt] = mfma32x32x16(va, ps[st2], os[dt]);
        }
      }
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
  lf += __shfl_xor(lf, 32, 64);
  if (STATS) {
    sink_l += __shfl_xor(sink_l, 32, 64);
    ex_l += __shfl_xor(ex_l, 32, 64);
  }
  ls += __shfl_xor(ls, 32, 64);
  const float inv_f = 1.f / lf, inv_s = 1.f / ls;
  const bool row_ok = qrow < qend;
  const int64_t row = static_cast<int64_t>(bh) * Nq + (qrow - q_off);
  float sq = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
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
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h_full) + row * kD + dcol) = u;
        }
        if (kSparse) {
          uint2 u = make_uint2(pack_bf16x2(hs[0], hs[1]), pack_bf16x2(hs[2], hs[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h_sparse) + row * kD + dcol) = u;
        }
      }
    }
  }
  if (MODE == kModeDual) sq += __shfl_xor(sq, 32, 64);
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
      a.sink_mass[row] = sink_l / lf;
      a.entropy[row] = kLn2 * (fast_log2(lf) - ex_l / lf);
    }
  }
}

template <int MODE, bool STATS>
void launch_mode(const Dims& D, const FwdArgs& a, size_t lds, int n_qtiles, float scale_log2, hipStream_t s) {
  static size_t granted = 0;    // LDS above 64 KiB in total must be requested per kernel
  if (lds > granted) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_mfma<MODE, STATS>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    granted = lds;
  }
  dim3 grid(D.B * D.Hq * n_qtiles);   // work items from qtile_item
  hipLaunchKernelGGL((k_fwd_mfma<MODE, STATS>), grid, dim3(256), lds, s, a, D.Hq, D.G, D.N, D.Nq, D.q_off, D.block,
                     D.nb, D.K,
                     scale_log2, n_qtiles);
}

constexpr size_t kStaticLds = 4 * kTile * sizeof(uint16_t);

size_t lds_bytes(const Dims& D) {   // dynamic part: selection bits
  const int W = (D.nb + 31) / 32;
  return static_cast<size_t>(kBM * W) * sizeof(uint32_t);
}

}  // namespace

bool fwd_mfma_supported(const Dims& D) {
  // the selection bits of 128 rows must fit in LDS next to the K/V tiles
  return D.dtype == 1 && D.d == kD && kStaticLds + lds_bytes(D) <= 160 * 1024;
}

void launch_fwd_mfma(const Dims& D, const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (D.Nq + kBM - 1) / kBM;
  const size_t lds = a.mode == kFullOnly ? 0 : lds_bytes(D);   // the full stream reads no selection bits
  const float scale_log2 = D.scale * 1.4426950408889634f;
  timing_begin(kKFwdMfma, s);
  const bool stats = a.sink_mass != nullptr;
  if (a.mode == kFullOnly) {
    if (stats) launch_mode<kModeFull, true>(D, a, lds, n_qtiles, scale_log2, s);
    else launch_mode<kModeFull, false>(D, a, lds, n_qtiles, scale_log2, s);
  } else {
    if (stats) launch_mode<kModeDual, true>(D, a, lds, n_qtiles, scale_log2, s);
    else launch_mode<kModeDual, false>(D, a, lds, n_qtiles, scale_log2, s);
  }
  timing_end(kKFwdMfma, s);
}

}  // namespace ssa
