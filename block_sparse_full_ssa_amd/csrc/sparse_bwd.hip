// Backward of SSA's sparse stream on key-block buckets, bf16 MFMA on gfx950.
//
// The sparse stream's gradient (Sintesi Tecnica, section 2: the stream
// gradient G_s of the sparse output through the softmax renormalised over
// each query's selected blocks) touches only the selected (query, key)
// pairs.  With the bucket of every (batch, KV head c, key block j) -- the
// rows of the G query heads of group c that selected j -- one workgroup per
// key block computes
//   P  = 2^(S c - lse_s)  on the block's keys (own block: keys <= t),
//   dS = P (G_s V^T - D_s),
//   dV_j = sum over the bucket of P^T G_s,   dK_j = scale sum of dS^T Q,
// over the gathered rows in batches of 32.  dK and dV of the block stay in
// registers over the whole bucket and are written once: as fp32 partials
// that the full-stream kernel adds (training modes), or as the bf16 result
// (sparse-only).  Keys of a block that no row selected get zero.  The
// stream's dQ = scale dS K leaves in one of two ways:
//   training modes: each entry's row of dS over the block's keys (bf16, in
//     the dQ kernel's lane order), which the query-stationary dQ kernel adds
//     to the full stream's dS, so that no atomics are needed;
//   sparse-only: each entry's partial dQ over the block's keys,
//     scale dS K_j (bf16, one row of d per bucket entry), which a merge
//     kernel adds up per query row over its selected blocks in selection
//     order: deterministic, and no atomics (fp32 atomics on this chip run at
//     a small fraction of the store bandwidth).
//
// Waves: wave w owns key half kh = w % KH (32 keys, B operands in registers)
// of query stream qs = w / KH; the 4 / KH streams take consecutive batches.
// Each stream's gathered Q and G_s rows move HBM -> LDS (one row per HD / 8
// lanes, double-buffered; HD, the head dimension 64 or 128, is a template
// parameter); dS^T of the block passes through LDS, where each
// wave reads back its own keys' rows for the dS rows, or, sparse-only, each
// wave of a stream reduces dQ over all the block's keys for its slice of d.
// The layout of every product is the full-stream kernel's (S = Q K^T, lane l
// owns key l % 32).

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

// Physical 16-byte chunk of logical chunk c: Q / G rows of 2 HD bytes (read by
// rows and by transposes), 64-byte dS^T rows.
// 256-byte rows (HD = 128): c ^ (2 (r % 8) + (r / 8) % 2), measured on gfx950
// to keep the transpose reads (ds_read_b64_tr_b16) free of bank conflicts as
// well as the 16-byte row reads, where c ^ (r % 8) or c ^ (r % 16) leave the
// transpose reads two-way conflicted.  128-byte rows (HD = 64): c ^ (r % 8).
template <int HD> __device__ __forceinline__ int swz_t(int r, int c) {
  return HD == 128 ? c ^ (((r & 7) << 1) | ((r >> 3) & 1)) : c ^ (r & 7);
}
__device__ __forceinline__ int swz_s(int r, int c) { return c ^ ((r >> 1) & 3); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

template <int KH, bool DSOUT, int HD>   // HD: head dimension
__global__ void __launch_bounds__(256, 1)
    k_bwd_sparse(SparseBwdArgs a, int Hq, int G, int N, int nb, float scale, float scale_log2) {
  constexpr int kD = HD;
  constexpr int kDT = HD / 32;               // 32-column tiles of dK / dV
  constexpr int kCh = HD / 8;                // 16-byte chunks per row
  constexpr int kBlk = 32 * KH;
  constexpr int QS = 4 / KH;                 // query streams
  constexpr int kT = 32 * kD;                // one Q / G tile
  constexpr int kDS = kBlk * 32;             // one dS^T tile
  // dQ columns per wave (sparse-only): a stream's waves split d, at least 32
  // columns each (HD = 64 with 128-key blocks: waves kh >= 2 have none)
  constexpr int kSlice = kD / KH >= 32 ? kD / KH : 32;
  // LDS: the key block (for the dQ operand), then per stream two sets of
  // {Q, G_s tiles, dS^T tile, row values}; separate objects per set so that
  // the compiler can tell the set being read from the one being filled
  __shared__ __attribute__((aligned(16))) uint16_t Kst[kBlk * kD];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QS * kT], Q1[QS * kT], F0[QS * kT], F1[QS * kT];
  __shared__ __attribute__((aligned(16))) uint16_t D0[QS * kDS], D1[QS * kDS];
  // row values per stream: lse2 [32], D [32], t [32] (int, -1: no row), 32 unused
  __shared__ __attribute__((aligned(16))) float R0[QS * 128], R1[QS * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave % KH, qs = wave / KH;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, li = lane & 15;
  const int gk = grp >> 1, sub16 = (grp & 1) * 16, srow = li >> 2, m4 = li & 3;

  const int bc = blockIdx.x, j = blockIdx.y;
  const int Hkv = Hq / G;
  const int b = bc / Hkv, c = bc % Hkv;
  const int64_t bucket = static_cast<int64_t>(bc) * nb + j;
  const int p0 = a.offs[bucket];
  const int n = a.offs[bucket + 1] - p0;
  const int32_t* list = a.rows + p0;
  const int kblk0 = j * kBlk;
  const int key = kblk0 + 32 * kh + col;      // this lane's key
  const int64_t kvbase = static_cast<int64_t>(bc) * N * kD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + kvbase;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + kvbase;
  const int64_t qhead0 = static_cast<int64_t>(b) * Hq + c * G;

  // result rows of the lane's key: d = 32 dt + 8 a4 + 4 g + e
  auto write_kv = [&](const f32x16* dk, const f32x16* dv) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * g;
        const int i = 4 * a4;
        const int64_t o = kvbase + static_cast<int64_t>(key) * kD + d0;
        if (a.dk_part) {
          *reinterpret_cast<float4*>(a.dk_part + o) =
              make_float4(scale * dk[dt][i], scale * dk[dt][i + 1], scale * dk[dt][i + 2], scale * dk[dt][i + 3]);
          *reinterpret_cast<float4*>(a.dv_part + o) = make_float4(dv[dt][i], dv[dt][i + 1], dv[dt][i + 2], dv[dt][i + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dk) + o) =
              make_uint2(pack_bf16x2(scale * dk[dt][i], scale * dk[dt][i + 1]),
                         pack_bf16x2(scale * dk[dt][i + 2], scale * dk[dt][i + 3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dv) + o) =
              make_uint2(pack_bf16x2(dv[dt][i], dv[dt][i + 1]), pack_bf16x2(dv[dt][i + 2], dv[dt][i + 3]));
        }
      }
  };

  f32x16 dv[kDT], dk[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dv[dt] = f32x16{};
    dk[dt] = f32x16{};
  }
  if (n == 0) {                                // nobody selected this block
    if (qs == 0) write_kv(dk, dv);
    return;
  }

  // ---- the key block in LDS (plain layout) for the dQ operand
  for (int e = tid; e < kBlk * kCh; e += 256) {
    const int row = e / kCh, c8 = e % kCh;
    *reinterpret_cast<uint4*>(&Kst[row * kD + 8 * c8]) =
        *reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(kblk0 + row) * kD + 8 * c8);
  }
  // S and dP B operands [16 d x 32 keys]: key = this lane's key, d = 16 ds + 8 g + s
  bf16x8 kb[kD / 16], vb[kD / 16];
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) {
    kb[ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(key) * kD + 16 * ds + 8 * g));
    vb[ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(key) * kD + 16 * ds + 8 * g));
  }
  __syncthreads();
  // dQ B operands [16 keys x 32 d]: d = slice + 32 dt + col, keys of k-step ks
  // in the transpose-read order of the dS^T tile
  constexpr int kDt = kSlice / 32;
  const bool has_slice = kSlice * kh < kD;    // uniform
  bf16x8 kq[DSOUT ? 1 : 2 * KH][kDt];
  if (!DSOUT && has_slice) {
#pragma unroll
    for (int ks = 0; ks < 2 * KH; ++ks)
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const uint16_t* p = &Kst[(16 * ks + 4 * gk + srow) * kD + kSlice * kh + 32 * dt + sub16 + 4 * m4];
        kq[ks][dt] = lds_tr_pair(p, p + 8 * kD);
      }
  }

  const int nbat = (n + 31) >> 5;
  const int iters = (nbat + QS - 1) / QS;
  // lane col's entry of the stream's batch bt (-1: none)
  auto entry = [&](int bt) -> int {
    const int idx = bt * 32 + col;
    return (bt < nbat && idx < n) ? list[idx] : -1;
  };
  auto row_of = [&](int e) -> int {
    if (e < 0) return 0;
    const int hl = e / N;
    return static_cast<int>((qhead0 + hl) * N + (e - hl * N));
  };
  // HBM -> LDS copy of the stream's Q and G_s rows of an entry set: 2 kOpsT
  // instructions of kRowsOp rows, split over the stream's KH waves; lane l
  // fills physical chunk l % kCh of row kRowsOp n + l / kCh
  constexpr int kRowsOp = 512 / HD, kOpsT = HD / 16;
  auto load_tiles = [&](int e, uint16_t* Qd, uint16_t* Fd) {
    const int R = row_of(e);
#pragma unroll
    for (int u = 0; u < 2 * kOpsT / KH; ++u) {
      const int nn = u * KH + kh;                 // uniform
      const int which = nn / kOpsT, n8 = nn % kOpsT;
      const int row = kRowsOp * n8 + lane / kCh;
      const int Rr = __shfl(R, row, 64);
      const uint16_t* src = which == 0 ? static_cast<const uint16_t*>(a.q) : a.g_sparse;
      uint16_t* dst = (which == 0 ? Qd : Fd) + qs * kT;
      const int cl = swz_t<HD>(row, lane % kCh);
      __builtin_amdgcn_global_load_lds((const glb_void*)(src + static_cast<int64_t>(Rr) * kD + 8 * cl),
                                       (lds_void*)(dst + n8 * 512), 16, 0, 0);
    }
  };
  // row values of an entry set, through registers (lanes 0..31 of wave kh = 0)
  float rv_lse = 0.f, rv_d = 0.f;
  int rv_t = -1, rv_r = 0;
  auto load_rows = [&](int e) {
    rv_t = -1;
    rv_r = 0;
    rv_lse = INFINITY;
    rv_d = 0.f;
    if (e >= 0) {
      const int hl = e / N;
      rv_t = e - hl * N;
      rv_r = row_of(e);
      rv_lse = a.lse2_sparse[rv_r];
      rv_d = a.D_sparse[rv_r];
    }
  };
  auto store_rows = [&](float* Rd) {
    if (kh == 0 && g == 0) {
      float* r = Rd + qs * 128;
      r[col] = rv_lse;
      r[32 + col] = rv_d;
      r[64 + col] = __int_as_float(rv_t);
    }
  };

  // one iteration on set (Q, F, dS, rv) while the next batch streams into (Qn, Fn, Rn)
  auto step = [&](int it, int e_next, const uint16_t* Q, const uint16_t* F, uint16_t* dS, const float* rv,
                  uint16_t* Qn, uint16_t* Fn, float* Rn) {
    const bool more = it + 1 < iters;
    if (more) {
      load_rows(e_next);
      load_tiles(e_next, Qn, Fn);
    }
    const bool has = it * QS + qs < nbat;                       // uniform
    const uint16_t* Qs = Q + qs * kT;
    const uint16_t* Fs = F + qs * kT;
    uint16_t* dSs = dS + qs * kDS;
    const float* rs = rv + qs * 128;
    // validity of the lane's 16 query rows for the dQ partials, taken before
    // the barrier (the row values are refilled after it)
    uint32_t rowok = 0u;
    if (has) {
      // ---- S = Q K^T, dP = G_s V^T [32 q x 32 keys]; lane: key col, queries 8(i/4)+4g+(i%4)
      f32x16 s = f32x16{}, dp = f32x16{};
      const int ra = col * kD;
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) {
        const int off = ra + 8 * swz_t<HD>(col, 2 * ds + g);
        s = mfma32x32x16(lds_read8(&Qs[off]), kb[ds], s);
        dp = mfma32x32x16(lds_read8(&Fs[off]), vb[ds], dp);
      }
      float p[16], dsv[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int qb = 8 * a4 + 4 * g;
        const float4 l4 = *reinterpret_cast<const float4*>(&rs[qb]);
        const float4 d4 = *reinterpret_cast<const float4*>(&rs[32 + qb]);
        const float4 t4 = *reinterpret_cast<const float4*>(&rs[64 + qb]);
        const float la[4] = {l4.x, l4.y, l4.z, l4.w}, da[4] = {d4.x, d4.y, d4.z, d4.w};
        const int ta[4] = {__float_as_int(t4.x), __float_as_int(t4.y), __float_as_int(t4.z), __float_as_int(t4.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * a4 + e;
          rowok |= ta[e] >= 0 ? (1u << i) : 0u;
          const bool live = key <= ta[e];                  // t = -1: no row
          p[i] = live ? fast_exp2(s[i] * scale_log2 - la[e]) : 0.f;
          dsv[i] = p[i] * (dp[i] - da[e]);
        }
      }
      // ---- dS^T -> LDS (bf16) for the dQ reduction over the block's keys
      {
        const int r = 32 * kh + col;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          uint2 u = make_uint2(pack_bf16x2(dsv[4 * a4], dsv[4 * a4 + 1]), pack_bf16x2(dsv[4 * a4 + 2], dsv[4 * a4 + 3]));
          *reinterpret_cast<uint2*>(&dSs[r * 32 + 8 * swz_s(r, a4) + 4 * g]) = u;
        }
      }
      if constexpr (DSOUT) {
        // ---- the rows of dS of this wave's 32 keys -> HBM for the query-
        // stationary dQ: the transposes of the wave's own dS^T rows for k-step
        // ks = 2 kh + h give lane (query col, g) element s = key 16 ks +
        // 8 (s / 4) + 4 g + s % 4.  A row of 32 keys is stored in the dQ
        // kernel's lane order, position 16 g' + 4 a + e for key 8 a + 4 g' + e,
        // so that element s of half h goes to position 16 g + 8 h + s.
        // (the transposes take all lanes: a lane's result holds other lanes' reads)
        uint4 u[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ks = 2 * kh + h;
          const int r0 = 16 * ks + 4 * gk + srow, r1 = r0 + 8;
          const int cl = 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
          u[h] = __builtin_bit_cast(
              uint4, lds_tr_pair(&dSs[r0 * 32 + 8 * swz_s(r0, cl) + e4], &dSs[r1 * 32 + 8 * swz_s(r1, cl) + e4]));
        }
        const int idx = (it * QS + qs) * 32 + col;
        if (idx < n) {
          uint16_t* dst = a.ds_rows + static_cast<int64_t>(p0 + idx) * kBlk + 32 * kh;
#pragma unroll
          for (int h = 0; h < 2; ++h) *reinterpret_cast<uint4*>(dst + 16 * g + 8 * h) = u[h];
        }
      }
      // ---- dV^T += G_s^T P, dK^T += Q^T dS  (k = queries; 2 steps of 16)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int o = 8 * st;
        const bf16x8 bp = to_bf16x8(p[o], p[o + 1], p[o + 2], p[o + 3], p[o + 4], p[o + 5], p[o + 6], p[o + 7]);
        const bf16x8 bds = to_bf16x8(dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3], dsv[o + 4], dsv[o + 5], dsv[o + 6], dsv[o + 7]);
        const int r0 = 16 * st + 4 * gk + srow, r1 = r0 + 8;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const int cl = 4 * dt + 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
          const int o0 = r0 * kD + 8 * swz_t<HD>(r0, cl) + e4, o1 = r1 * kD + 8 * swz_t<HD>(r1, cl) + e4;
          dv[dt] = mfma32x32x16(lds_tr_pair(&Fs[o0], &Fs[o1]), bp, dv[dt]);
          dk[dt] = mfma32x32x16(lds_tr_pair(&Qs[o0], &Qs[o1]), bds, dk[dt]);
        }
      }
    }
    if (more) store_rows(Rn);
    __builtin_amdgcn_s_waitcnt(0);     // next tiles landed, dS^T written
    __syncthreads();

    // ---- dQ[32 q x slice] of the stream's batch = dS[32 q x block keys] K[block keys x slice]
    if (!DSOUT && has && has_slice) {
      f32x16 dq[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) dq[dt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2 * KH; ++ks) {
        const int r0 = 16 * ks + 4 * gk + srow, r1 = r0 + 8;
        const int cl = 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
        const bf16x8 ds_op =
            lds_tr_pair(&dSs[r0 * 32 + 8 * swz_s(r0, cl) + e4], &dSs[r1 * 32 + 8 * swz_s(r1, cl) + e4]);
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) dq[dt] = mfma32x32x16(ds_op, kq[ks][dt], dq[dt]);
      }
      // the batch's entries are p0 + 32 bt + r (r: the query of register i)
      const int64_t e0 = static_cast<int64_t>(p0) + (it * QS + qs) * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!((rowok >> i) & 1u)) continue;
        const int r = 8 * (i >> 2) + 4 * g + (i & 3);
        uint16_t* dst = a.dq_part + (e0 + r) * kD + kSlice * kh + col;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) dst[32 * dt] = to_bf16(scale * dq[dt][i]).bits;
      }
    }
  };

  // prologue: the first batch of every stream
  int e_cur = entry(qs);
  load_rows(e_cur);
  load_tiles(e_cur, Q0, F0);
  store_rows(R0);
  int e_next = entry(QS + qs);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < iters; it += 2) {
    int e_after = entry((it + 2) * QS + qs);
    step(it, e_next, Q0, F0, D0, R0, Q1, F1, R1);
    e_next = e_after;
    if (it + 1 >= iters) break;
    e_after = entry((it + 3) * QS + qs);
    step(it + 1, e_next, Q1, F1, D1, R1, Q0, F0, R0);
    e_next = e_after;
  }

  // ---- reduce dK / dV over the streams of each key half (one stream and
  // one tensor at a time through 16 KiB of the free Q tiles: Q0 for key
  // half 0, Q1 for key half 1), then write
  if (QS > 1) {
    float* red = reinterpret_cast<float*>(kh == 0 ? Q0 : Q1);
    for (int o = 1; o < QS; ++o) {
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        f32x16* acc = part == 0 ? dk : dv;
        __syncthreads();
        if (qs == o) {
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[(dt * 16 + i) * 64 + lane] = acc[dt][i];
        }
        __syncthreads();
        if (qs == 0) {
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[dt][i] += red[(dt * 16 + i) * 64 + lane];
        }
      }
    }
  }
  if (qs == 0) write_kv(dk, dv);
}

// Sparse-only dQ: the sum of a query row's partials over its selected
// blocks, in selection order.  LR = HD / 8 lanes per row (8 columns of d
// each), 256 / LR rows per workgroup; the partial of (row, block j) is the
// row's entry in bucket (b, c, j), found through the bucket mask word and its
// position.  Entries naming no causal block, and repeats, are skipped (no
// partial).
template <int HD>
__global__ void __launch_bounds__(256) k_sparse_dq_merge(const int32_t* __restrict__ sel,
                                                         const uint32_t* __restrict__ mask,
                                                         const int32_t* __restrict__ wpos,
                                                         const uint16_t* __restrict__ part, void* dq, int64_t rows,
                                                         int Hq, int G, int N, int block, int nb, int K, int Kc) {
  constexpr int kD = HD, LR = HD / 8;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / LR) + (threadIdx.x / LR);
  const int li = threadIdx.x % LR;
  const bool live = row < rows;
  const int64_t rr = live ? row : 0;
  const int64_t bh = rr / N;
  const int t = static_cast<int>(rr - bh * N);
  const int b = static_cast<int>(bh / Hq), h = static_cast<int>(bh % Hq);
  const int Hkv = Hq / G, nqt = N / 32;
  const int64_t bc = static_cast<int64_t>(b) * Hkv + h / G;
  const int hl = h % G, qt = t >> 5;
  const uint32_t below = (1u << (t & 31)) - 1u;
  const int own = t / block;
  const int32_t* s = sel + rr * K;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int e0 = 0; e0 < Kc; e0 += LR) {
    // lane li looks up slot e0 + li; the LR lanes then take the slots in order
    const int e = e0 + li;
    int j = (live && e < Kc) ? s[e] : -1;
    if (j > own || (e > 0 && j >= 0 && s[e - 1] == j)) j = -1;
    int64_t p = 0;
    if (j >= 0) {
      const int64_t w = ((bc * nb + j) * G + hl) * nqt + qt;
      p = wpos[w] + __popc(mask[w] & below);
    }
    const int nslot = min(LR, Kc - e0);
    for (int i = 0; i < nslot; ++i) {
      const int ji = __shfl(j, i, LR);
      if (ji < 0) continue;
      const uint32_t plo = __shfl(static_cast<uint32_t>(p), i, LR);
      const uint32_t phi = __shfl(static_cast<uint32_t>(p >> 32), i, LR);
      const int64_t pi = (static_cast<int64_t>(phi) << 32) | plo;
      const uint4 u = *reinterpret_cast<const uint4*>(part + pi * kD + 8 * li);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        acc[2 * k2] += __uint_as_float(wd[k2] << 16);
        acc[2 * k2 + 1] += __uint_as_float(wd[k2] & 0xffff0000u);
      }
    }
  }
  if (!live) return;
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dq) + row * kD + 8 * li) = o;
}

}  // namespace

void launch_sparse_dq_merge(const Dims& D, const int32_t* sel, const uint32_t* mask, const int32_t* wpos,
                            const uint16_t* part, void* dq, hipStream_t s) {
  const int Kc = D.K < D.nb ? D.K : D.nb;
  const int rows_wg = 256 / (D.d / 8);
  const dim3 grid(static_cast<unsigned>((D.rows() + rows_wg - 1) / rows_wg));
  timing_begin(kKDqMerge, s);
  if (D.d == 64)
    hipLaunchKernelGGL(k_sparse_dq_merge<64>, grid, dim3(256), 0, s, sel, mask, wpos, part, dq, D.rows(), D.Hq, D.G,
                       D.N, D.block, D.nb, D.K, Kc);
  else
    hipLaunchKernelGGL(k_sparse_dq_merge<128>, grid, dim3(256), 0, s, sel, mask, wpos, part, dq, D.rows(), D.Hq, D.G,
                       D.N, D.block, D.nb, D.K, Kc);
  timing_end(kKDqMerge, s);
}

bool sparse_bwd_supported(const Dims& D) { return D.dtype == 1 && (D.d == 128 || D.d == 64); }

void launch_bwd_sparse(const Dims& D, const SparseBwdArgs& a, hipStream_t s) {
  dim3 grid(D.B * D.Hkv, D.nb);
  const float scale_log2 = D.scale * 1.4426950408889634f;
  timing_begin(kKBwdSparse, s);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.nb, D.scale, scale_log2);
  };
  const bool rows_out = a.ds_rows != nullptr;
  auto by_block = [&](auto hd_tag) {
    constexpr int HD = decltype(hd_tag)::value;
    if (D.block == 32) rows_out ? go(k_bwd_sparse<1, true, HD>) : go(k_bwd_sparse<1, false, HD>);
    else if (D.block == 64) rows_out ? go(k_bwd_sparse<2, true, HD>) : go(k_bwd_sparse<2, false, HD>);
    else rows_out ? go(k_bwd_sparse<4, true, HD>) : go(k_bwd_sparse<4, false, HD>);
  };
  if (D.d == 64) by_block(std::integral_constant<int, 64>{});
  else by_block(std::integral_constant<int, 128>{});
  timing_end(kKBwdSparse, s);
}

}  // namespace ssa
