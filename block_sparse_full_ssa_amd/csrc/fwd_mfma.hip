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
// S^T accumulator) keeps the output of query l % 32 in lane l.
//
// Sparse stream: P_sparse = P_full * 2^(m_full - m_sparse) on selected key
// blocks (one multiply instead of a second exponential) whenever that factor
// is at most 2^64 for every lane of the wave; otherwise the exponential is
// evaluated directly.  When every block is selected the two streams execute
// identical operations and their outputs agree bit for bit.

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kD = 128;        // head dimension
constexpr int kBM = 128;       // queries per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kKPitch = 136;   // K tile row pitch (elements), padded against bank conflicts
constexpr int kVPitch = 128;   // V tile row pitch (read with transpose reads)
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTau = 8.f;    // lazy-rescale threshold (log2 units)

enum { kModeDual = 0, kModeFull = 1, kModeSparse = 2 };

template <int MODE>
__global__ void __launch_bounds__(256, 1)
    k_fwd_mfma(FwdArgs a, int Hq, int G, int N, int block, int nb, int K, float scale_log2, int n_qtiles) {
  // dynamic LDS: K tiles [2][64][136], V tiles [2][64][128], then the
  // selection bits [kBM][W] of the rows and their union [W]
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Kbuf = lds;
  uint16_t* Vbuf = lds + 2 * kBN * kKPitch;
  uint32_t* bits = reinterpret_cast<uint32_t*>(lds + 2 * kBN * kKPitch + 2 * kBN * kVPitch);
  const int W = (nb + 31) >> 5;
  uint32_t* anybits = bits + kBM * W;

  const int tid = threadIdx.x;
  // The wave index and every condition that guards an MFMA are made
  // wave-uniform for the compiler (readfirstlane): matrix instructions must
  // sit behind scalar branches, never behind an EXEC mask.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x;
  const int q0 = (n_qtiles - 1 - static_cast<int>(blockIdx.y)) * kBM;   // longest tiles first
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(bh) * N * kD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + bc * N * kD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + bc * N * kD;

  // ---- selection bits of the workgroup's rows
  if (MODE != kModeFull) {
    for (int e = tid; e < kBM * W + W; e += 256) bits[e] = 0u;
    __syncthreads();
    for (int e = tid; e < kBM * K; e += 256) {
      const int r = e / K, t = q0 + r;
      if (t < N) {
        const int blk = a.sel[(static_cast<int64_t>(bh) * N + t) * K + (e - r * K)];
        if (blk >= 0) {
          atomicOr(&bits[r * W + (blk >> 5)], 1u << (blk & 31));
          atomicOr(&anybits[blk >> 5], 1u << (blk & 31));
        }
      }
    }
  }

  // ---- the wave's 32 queries as B operands (query = col, d = 16*ds + 8*g + s)
  const int qrow = q0 + wave * 32 + col;           // this lane's query
  const bool wave_live = q0 + wave * 32 < N;
  const int wave_last_q = min(N - 1, q0 + wave * 32 + 31);
  bf16x8 qreg[kD / 16];
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < N) u = *reinterpret_cast<const uint4*>(qg + static_cast<int64_t>(qrow) * kD + 16 * ds + 8 * g);
    qreg[ds] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 of[4], os[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    of[dt] = f32x16{};
    os[dt] = f32x16{};
  }
  float mf = -INFINITY, lf = 0.f, ms = -INFINITY, ls = 0.f;

  const int j_last = min(N - 1, q0 + kBM - 1) / kBN;
  if (MODE != kModeFull) __syncthreads();

  // tile needed by the workgroup? (sparse-only mode skips unselected tiles)
  auto tile_needed = [&](int j) -> bool {
    if (MODE != kModeSparse) return true;
    const int b0 = (j * kBN) / block, b1 = (j * kBN + kBN - 1) / block;
    for (int bb = b0; bb <= b1 && bb < nb; ++bb)
      if ((anybits[bb >> 5] >> (bb & 31)) & 1u) return true;
    return false;
  };
  auto next_tile = [&](int j) -> int {
    for (++j; j <= j_last; ++j)
      if (tile_needed(j)) return j;
    return j_last + 1;
  };

  // global -> register prefetch of one K/V tile: thread owns chunks tid + 256 r
  uint4 kpre[4], vpre[4];
  auto prefetch = [&](int j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + 256 * r, row = c >> 4, c8 = c & 15;
      const int key = j * kBN + row;
      if (key < N) {
        kpre[r] = *reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(key) * kD + 8 * c8);
        vpre[r] = *reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(key) * kD + 8 * c8);
      } else {
        kpre[r] = make_uint4(0, 0, 0, 0);
        vpre[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + 256 * r, row = c >> 4, c8 = c & 15;
      *reinterpret_cast<uint4*>(&Kbuf[buf * kBN * kKPitch + row * kKPitch + 8 * c8]) = kpre[r];
      *reinterpret_cast<uint4*>(&Vbuf[buf * kBN * kVPitch + row * kVPitch + 8 * c8]) = vpre[r];
    }
  };

  // Double-buffered K/V: tile j is read from buffer `cur` while tile jn is
  // loaded into registers and then written to the other buffer; one barrier
  // per tile.
  int j = MODE == kModeSparse ? next_tile(-1) : 0;
  int cur = 0;
  if (j <= j_last) {
    prefetch(j);
    stage(0);
  }
  __syncthreads();
  while (j <= j_last) {
    const uint16_t* Ks = Kbuf + cur * kBN * kKPitch;
    const uint16_t* Vs = Vbuf + cur * kBN * kVPitch;
    const int jn = MODE == kModeSparse ? next_tile(j) : j + 1;
    if (jn <= j_last) prefetch(jn);

    // ---- selection of this tile's (one or two) key blocks for the lane's query
    bool sb[2] = {false, false};
    bool sparse_any = false;
    const bool wave_in = wave_live && j * kBN <= wave_last_q;
    if (MODE != kModeFull && wave_in) {
      const int r = wave * 32 + col;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int blk = (j * kBN + kh * 32) / block;
        sb[kh] = qrow < N && blk < nb && ((bits[r * W + (blk >> 5)] >> (blk & 31)) & 1u);
      }
      sparse_any = __builtin_amdgcn_readfirstlane(__any(sb[0] || sb[1]) ? 1 : 0) != 0;
    }

    if (wave_in && (MODE != kModeSparse || sparse_any)) {
      // ---- S^T = K Q^T for the two 32-key halves
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          bf16x8 ka = lds_read8(&Ks[(kh * 32 + col) * kKPitch + 16 * ds + 8 * g]);
          s[kh] = mfma32x32x16(ka, qreg[ds], s[kh]);
        }
      }
      // ---- scale to log2 units, causal mask near the diagonal
      const bool diag = j * kBN + kBN - 1 > q0 + wave * 32;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[kh][i] * scale_log2;
          if (diag) {
            const int key = j * kBN + kh * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > qrow) x = -INFINITY;
          }
          s[kh][i] = x;
        }
      }
      float mx[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float m = s[kh][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, s[kh][i]);
        mx[kh] = fmaxf(m, __shfl_xor(m, 32, 64));
      }

      // lazy rescaling: the running maximum moves only when a tile exceeds it
      // by more than kTau (log2 units), so probabilities stay below 2^kTau
      const float mxf = fmaxf(mx[0], mx[1]);
      const float mfn = MODE != kModeSparse ? (mxf > mf + kTau ? mxf : mf) : 0.f;
      float pv[2][16];
      float msn = ms, sum_s = 0.f;
      bool rescale = false;
      if (MODE != kModeFull && sparse_any) {
        const float mxs = fmaxf(sb[0] ? mx[0] : -INFINITY, sb[1] ? mx[1] : -INFINITY);
        msn = mxs > ms + kTau ? mxs : ms;
        // dual mode: derive P_sparse from P_full when 2^(m_full - m_sparse) is safe
        rescale = MODE == kModeDual && !__any((sb[0] || sb[1]) && (mfn - msn > 64.f));
        if (!rescale) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = sb[kh] ? fast_exp2(s[kh][i] - msn) : 0.f;
              pv[kh][i] = p;
              sum_s += p;
            }
        }
      }

      bf16x8 pf[4], ps[4];
      if (MODE != kModeSparse) {
        // full stream
        const float alpha = fast_exp2(mf - mfn);
        float sum = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(s[kh][i] - mfn);
            s[kh][i] = p;
            sum += p;
          }
        lf = lf * alpha + sum;
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) of[dt] *= alpha;
        }
        mf = mfn;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kh = st >> 1, o = 8 * (st & 1);
          pf[st] = to_bf16x8(s[kh][o], s[kh][o + 1], s[kh][o + 2], s[kh][o + 3], s[kh][o + 4], s[kh][o + 5],
                             s[kh][o + 6], s[kh][o + 7]);
        }
      }
      if (MODE != kModeFull && sparse_any) {
        if (rescale) {
          const float c = (sb[0] || sb[1]) ? fast_exp2(mfn - msn) : 0.f;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = sb[kh] ? s[kh][i] * c : 0.f;
              pv[kh][i] = p;
              sum_s += p;
            }
        }
        const float alpha_s = msn == -INFINITY ? 1.f : fast_exp2(ms - msn);
        ls = ls * alpha_s + sum_s;
        if (__any(alpha_s != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) os[dt] *= alpha_s;
        }
        ms = msn;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kh = st >> 1, o = 8 * (st & 1);
          ps[st] = to_bf16x8(pv[kh][o], pv[kh][o + 1], pv[kh][o + 2], pv[kh][o + 3], pv[kh][o + 4],
                             pv[kh][o + 5], pv[kh][o + 6], pv[kh][o + 7]);
        }
      }

      // ---- O^T += V^T P^T; V^T operand through transpose reads
      const bool do_full = MODE != kModeSparse;
      const bool do_sparse = MODE != kModeFull && sparse_any;
      const int grp = lane >> 4, li = lane & 15;
      const int dsub = (grp & 1) * 16, gk = grp >> 1;   // d half and key group of this 16-lane group
      const int srow = li >> 2, m4 = li & 3;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint16_t* r0 = &Vs[(16 * st + 4 * gk + srow) * kVPitch + dsub + 4 * m4];
        const uint16_t* r1 = r0 + 8 * kVPitch;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          bf16x8 va = lds_tr_pair(r0 + 32 * dt, r1 + 32 * dt);
          if (do_full) of[dt] = mfma32x32x16(va, pf[st], of[dt]);
          if (do_sparse) os[dt] = mfma32x32x16(va, ps[st], os[dt]);
        }
      }
    }
    if (jn <= j_last) stage(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    j = jn;
  }

  // ---- epilogue
  if (!wave_live) return;
  lf += __shfl_xor(lf, 32, 64);
  ls += __shfl_xor(ls, 32, 64);
  const float inv_f = 1.f / lf, inv_s = 1.f / ls;
  const bool row_ok = qrow < N;
  const int64_t row = static_cast<int64_t>(bh) * N + qrow;
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
        if (MODE != kModeSparse) {
          uint2 u = make_uint2(pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h_full) + row * kD + dcol) = u;
        }
        if (MODE != kModeFull) {
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
    if (MODE != kModeSparse && a.lse_full) a.lse_full[row] = lse_f;
    if (MODE != kModeFull && a.lse_sparse) a.lse_sparse[row] = lse_s;
    if (MODE == kModeDual) {
      a.delta[row] = -expm1f(lse_s - lse_f);
      a.row_sq[row] = sq;
    }
  }
}

}  // namespace

size_t fwd_mfma_lds_bytes(const Dims& D);

bool fwd_mfma_supported(const Dims& D) {
  // the selection bits of 128 rows must fit in LDS next to the K/V tiles
  return D.dtype == 1 && D.d == kD && fwd_mfma_lds_bytes(D) <= 160 * 1024;
}

template <int MODE>
static void launch_mode(const Dims& D, const FwdArgs& a, size_t lds, int n_qtiles, float scale_log2,
                        hipStream_t s) {
  static size_t granted = 0;    // dynamic LDS above 64 KiB must be requested per kernel
  if (lds > granted) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_mfma<MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    granted = lds;
  }
  dim3 grid(D.B * D.Hq, n_qtiles);
  hipLaunchKernelGGL(k_fwd_mfma<MODE>, grid, dim3(256), lds, s, a, D.Hq, D.G, D.N, D.block, D.nb, D.K,
                     scale_log2, n_qtiles);
}

size_t fwd_mfma_lds_bytes(const Dims& D) {
  const int W = (D.nb + 31) / 32;
  return static_cast<size_t>(2 * kBN * kKPitch + 2 * kBN * kVPitch) * sizeof(uint16_t) +
         static_cast<size_t>(kBM * W + W) * sizeof(uint32_t);
}

void launch_fwd_mfma(const Dims& D, const FwdArgs& a, hipStream_t s) {
  const int n_qtiles = (D.N + kBM - 1) / kBM;
  const size_t lds = fwd_mfma_lds_bytes(D);
  const float scale_log2 = D.scale * 1.4426950408889634f;
  timing_begin(kKFwdMfma, s);
  if (a.mode == kFullOnly) launch_mode<kModeFull>(D, a, lds, n_qtiles, scale_log2, s);
  else if (a.mode == kSparseOnly) launch_mode<kModeSparse>(D, a, lds, n_qtiles, scale_log2, s);
  else launch_mode<kModeDual>(D, a, lds, n_qtiles, scale_log2, s);
  timing_end(kKFwdMfma, s);
}

}  // namespace ssa
