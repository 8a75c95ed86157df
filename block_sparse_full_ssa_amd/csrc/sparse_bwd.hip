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
// Waves: 2 KH per workgroup, wave w owns key half kh = w % KH (32 keys) in
// role w / KH.  Role 0 computes S = Q K^T (K rows of its keys as B operands
// in registers), P, and accumulates dV; role 1 computes dP = G_s V^T (V rows
// in registers), takes P from role 0 through LDS after a barrier, forms dS
// and accumulates dK.  Each wave so holds one accumulator and one operand
// set, which keeps it within half the register file: two workgroups (two
// waves per SIMD) share a CU.  The batch's gathered Q and G_s rows move HBM ->
// LDS (one row per HD / 8 lanes, double-buffered; HD, the head dimension 64
// or 128, is a template parameter); dS^T of the block passes through LDS,
// where each role-1 wave reads back its own keys' rows for the dS rows, or,
// sparse-only, every wave reduces dQ over all the block's keys for its slice
// of d.  The layout of every product is the full-stream kernel's (S = Q K^T,
// lane l owns key l % 32).

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

// Physical 16-byte chunk of logical chunk c: Q / G rows of 2 HD bytes (read by
// rows and by transposes), 64-byte dS^T rows.
// swz256 for 256-byte rows (HD = 128), swz128 for 128-byte rows (HD = 64).
template <int HD> __device__ __forceinline__ int swz_t(int r, int c) {
  return HD == 128 ? swz256(r, c) : swz128(r, c);
}
__device__ __forceinline__ int swz_s(int r, int c) { return c ^ ((r >> 1) & 3); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Barrier for LDS data only: memory operations in flight (the next batch's
// rows) are not waited for, as a plain __syncthreads would.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int KH, bool DSOUT, int HD>   // HD: head dimension
__global__ void __launch_bounds__(128 * KH, 2)
    k_bwd_sparse(SparseBwdArgs a, int Hq, int G, int N, int nb, float scale, float scale_log2) {
  constexpr int kD = HD;
  constexpr int kDT = HD / 32;               // 32-column tiles of dK / dV
  constexpr int kCh = HD / 8;                // 16-byte chunks per row
  constexpr int kBlk = 32 * KH;
  constexpr int kW = 2 * KH;                 // waves: (key half, role)
  constexpr int kT = 32 * kD;                // one Q / G tile
  constexpr int kDS = kBlk * 32;             // one dS^T tile
  // dQ columns per wave (sparse-only): the waves split d, at least 32
  // columns each (waves past the end of d have none)
  constexpr int kSlice = kD / kW >= 32 ? kD / kW : 32;
  // LDS: the key block (for the dQ operand), two sets of {Q, G_s tiles, row
  // values} (one being read while the next batch's is filled), the dS^T tile
  // and each key half's P
  __shared__ __attribute__((aligned(16))) uint16_t Kst[kBlk * kD];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[kT], Q1[kT], F0[kT], F1[kT];
  __shared__ __attribute__((aligned(16))) uint16_t DS[kDS];
  __shared__ __attribute__((aligned(16))) float PX[KH * 1024];
  // row values: lse2 [32], D [32], t [32] (int, -1: no row), 32 unused
  __shared__ __attribute__((aligned(16))) float R0[128], R1[128];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave % KH, role = wave / KH;   // role 0: S, P, dV; role 1: dP, dS, dK
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

  // the wave's result rows of the lane's key (dV for role 0, dK for role 1):
  // d = 32 dt + 8 a4 + 4 g + e
  auto write_out = [&](const f32x16* acc) {
    const float f = role ? scale : 1.f;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * g;
        const int i = 4 * a4;
        const int64_t o = kvbase + static_cast<int64_t>(key) * kD + d0;
        if (a.dk_part) {
          *reinterpret_cast<float4*>((role ? a.dk_part : a.dv_part) + o) =
              make_float4(f * acc[dt][i], f * acc[dt][i + 1], f * acc[dt][i + 2], f * acc[dt][i + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(role ? a.dk : a.dv) + o) =
              make_uint2(pack_bf16x2(f * acc[dt][i], f * acc[dt][i + 1]),
                         pack_bf16x2(f * acc[dt][i + 2], f * acc[dt][i + 3]));
        }
      }
  };

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16{};
  if (n == 0) {                                // nobody selected this block
    write_out(acc);
    return;
  }

  // ---- the key block in LDS (plain layout) for the dQ operand
  if constexpr (!DSOUT) {
    for (int e = tid; e < kBlk * kCh; e += 64 * kW) {
      const int row = e / kCh, c8 = e % kCh;
      *reinterpret_cast<uint4*>(&Kst[row * kD + 8 * c8]) =
          *reinterpret_cast<const uint4*>(kg + static_cast<int64_t>(kblk0 + row) * kD + 8 * c8);
    }
  }
  // B operand [16 d x 32 keys] of S (role 0: K) or dP (role 1: V): key = this
  // lane's key, d = 16 ds + 8 g + s
  bf16x8 kvb[kD / 16];
  {
    const uint16_t* src = (role ? vg : kg) + static_cast<int64_t>(key) * kD + 8 * g;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) kvb[ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + 16 * ds));
  }
  __syncthreads();
  // dQ B operands [16 keys x 32 d]: d = slice + 32 dt + col, keys of k-step ks
  // in the transpose-read order of the dS^T tile
  constexpr int kDt = kSlice / 32;
  const bool has_slice = kSlice * wave < kD;   // uniform
  bf16x8 kq[DSOUT ? 1 : 2 * KH][kDt];
  if (!DSOUT && has_slice) {
#pragma unroll
    for (int ks = 0; ks < 2 * KH; ++ks)
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const uint16_t* p = &Kst[(16 * ks + 4 * gk + srow) * kD + kSlice * wave + 32 * dt + sub16 + 4 * m4];
        kq[ks][dt] = lds_tr_pair(p, p + 8 * kD);
      }
  }

  const int nbat = (n + 31) >> 5;
  // Lane col's entry of batch bt, loaded unconditionally (past the bucket's
  // end: its last entry) so that every batch issues the same memory
  // instructions, and whether it is one of the bucket's: the loaded value is
  // combined with nothing before its use a batch later, so that the compiler
  // does not wait for the load as soon as it is issued.
  auto entry = [&](int bt) -> int { return list[min(bt * 32 + col, n - 1)]; };
  auto live = [&](int bt) -> bool { return bt * 32 + col < n; };
  auto row_of = [&](int e, bool ok) -> int {
    const int hl = ok ? e / N : 0;
    return ok ? static_cast<int>((qhead0 + hl) * N + (e - hl * N)) : 0;
  };
  // The Q and G_s rows of an entry set: 2 kOpsT 16-byte copies of kRowsOp
  // rows, split over the kW waves; lane l takes physical chunk l % kCh of
  // row kRowsOp n + l / kCh.  Training modes copy HBM -> LDS directly at the
  // start of a batch, into the other of two separately declared tile sets
  // (with the loop unrolled twice, the compiler can tell the set being filled
  // from the one being read).  Sparse-only, whose dQ products need more
  // registers, goes through registers: loads at the start of a batch, LDS
  // stores at its end, in a loop that is not unrolled (measured faster there,
  // and the twice-unrolled form spills).
  constexpr int kRowsOp = 512 / HD, kOpsT = HD / 16;
  static_assert((2 * kOpsT) % kW == 0, "tile copies must split evenly over the waves");
  constexpr int kPer = 2 * kOpsT / kW;
  auto copy_src = [&](int R, int u) {
    const int nn = u * kW + wave;               // uniform
    const int which = nn / kOpsT, n8 = nn % kOpsT;
    const int row = kRowsOp * n8 + lane / kCh;
    const int Rr = __shfl(R, row, 64);
    const uint16_t* src = which == 0 ? static_cast<const uint16_t*>(a.q) : a.g_sparse;
    return src + static_cast<int64_t>(Rr) * kD + 8 * swz_t<HD>(row, lane % kCh);
  };
  auto copy_dst = [&](uint16_t* Qd, uint16_t* Fd, int u) {
    const int nn = u * kW + wave;
    return (nn / kOpsT == 0 ? Qd : Fd) + (nn % kOpsT) * 512;
  };
  u32x4 pre[DSOUT ? 1 : kPer];
  // The copies' address registers stay allocated until the end of the batch:
  // an LDS read into a register that a copy in flight takes its address from
  // makes the compiler wait for every load and copy, the prefetch included.
  const uint16_t* src_of[kPer];
  auto load_tiles = [&](int e, bool ok, uint16_t* Qd, uint16_t* Fd) {
    const int R = row_of(e, ok);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      src_of[u] = copy_src(R, u);
      if constexpr (DSOUT)
        __builtin_amdgcn_global_load_lds((const glb_void*)src_of[u], (lds_void*)copy_dst(Qd, Fd, u), 16, 0, 0);
      else
        pre[u] = *reinterpret_cast<const u32x4*>(src_of[u]);
    }
  };
  auto hold_sources = [&]() {
#pragma unroll
    for (int u = 0; u < kPer; ++u) asm volatile("" ::"v"(src_of[u]));
  };
  auto store_tiles = [&](uint16_t* Qd, uint16_t* Fd) {
    if constexpr (!DSOUT) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) *reinterpret_cast<u32x4*>(copy_dst(Qd, Fd, u) + 8 * lane) = pre[u];
    }
  };
  // row values of an entry set, through registers (lanes 0..31 of wave 0)
  // (loaded unconditionally as well; a row past the bucket's end stores
  // lse = inf, D = 0, t = -1)
  float rv_lse = 0.f, rv_d = 0.f;
  int rv_t = -1;
  auto load_rows = [&](int e, bool ok) {
    if (wave == 0) {
      const int r = row_of(e, ok);
      rv_lse = a.lse2_sparse[r];
      rv_d = a.D_sparse[r];
      rv_t = ok ? e - (e / N) * N : -1;
    }
  };
  auto store_rows = [&](float* Rd, bool ok) {
    if (wave == 0 && g == 0) {
      Rd[col] = ok ? rv_lse : INFINITY;
      Rd[32 + col] = ok ? rv_d : 0.f;
      Rd[64 + col] = __int_as_float(rv_t);
    }
  };

  // P of the lane's 16 queries, element-major so that each access is one
  // contiguous 1 KiB row of the key half's buffer
  float* px = PX + kh * 1024 + lane * 4;

  // one batch on set (Q, F, rv) while the next batch streams into (Qn, Fn, Rn)
  auto step = [&](int it, int e_next, const uint16_t* Qs, const uint16_t* Fs, const float* rs, uint16_t* Qn,
                  uint16_t* Fn, float* Rn) {
    const bool more = it + 1 < nbat;
    const bool ok_next = live(it + 1);
    if (more) {
      load_rows(e_next, ok_next);
      load_tiles(e_next, ok_next, Qn, Fn);
    }
    // The lane parts of the LDS offsets, opaque to the compiler in each
    // batch: otherwise it keeps every offset of both tile sets in registers
    // across the loop and the wave no longer fits half the register file.
    int cx = col, rx = 4 * gk + srow, cq = 2 * (grp & 1) + (m4 >> 1);
    asm volatile("" : "+v"(cx), "+v"(rx), "+v"(cq));
    const int e4 = 4 * (m4 & 1);
    // Byte offsets, built once per batch from those lane parts.  Row reads of
    // d-step ds (row cx): the first half computed, d-step ds + kRO flipping
    // one bit (its logical chunk 2 ds + g flips the top bit, and so does the
    // physical one: bit 7 at HD = 128, bit 6 at HD = 64).  Transposes of
    // k-step st and d tile dt (rows 16 st + rx and 8 below): logical chunk
    // 4 dt + cq of a row whose swizzle term is 4 t + rx / 4 (+ 2), t = rx % 4
    // (HD = 128) or (rx % 4) / 2 % 2 (HD = 64), sits at 4 (dt ^ t) + (cq ^
    // (rx / 4 (+ 2))); the term 32 t is kept on bits the rest leaves clear,
    // so dt is an XOR of 64 dt and st a constant.
    constexpr int kRO = kD / 32;
    int ro[kRO];
#pragma unroll
    for (int ds = 0; ds < kRO; ++ds) ro[ds] = 2 * (cx * kD + 8 * swz_t<HD>(cx, 2 * ds + g));
    const int tt = HD == 128 ? (rx & 3) : ((rx & 3) >> 1) & 1;
    const int tb0 = 2 * (rx * kD + 8 * (cq ^ (rx >> 2)) + e4 + 32 * tt);
    const int tb1 = 2 * ((rx + 8) * kD + 8 * (cq ^ ((rx >> 2) + 2)) + e4 + 32 * tt);
    auto at = [](const uint16_t* T, int off) {
      return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(T) + off);
    };
    // A operand [32 q x 16 d] of S / dP (k-step ds) from a Q / G_s tile
    auto rdA = [&](const uint16_t* T, int ds) { return lds_read8(at(T, ds < kRO ? ro[ds] : ro[ds - kRO] ^ kD)); };
    // A operand [32 d x 16 q] (transposed tile, k-step st, d tile dt)
    auto rdT = [&](const uint16_t* T, int st, int dt) {
      return lds_tr_pair(at(T, (tb0 ^ (64 * dt)) + 32 * kD * st), at(T, (tb1 ^ (64 * dt)) + 32 * kD * st));
    };
    // transposing read of the dS^T tile for k-step ks (keys 16 ks ..)
    auto rdS = [&](int ks) {
      const int r0 = 16 * ks + rx, r1 = r0 + 8;
      return lds_tr_pair(&DS[r0 * 32 + 8 * swz_s(r0, cq) + e4], &DS[r1 * 32 + 8 * swz_s(r1, cq) + e4]);
    };
    // the lane's 16 query rows (queries 8(i/4)+4g+(i%4)): bit i of rowok says
    // the row exists (t >= 0), bit i of causal that the lane's key is <= t
    uint32_t rowok = 0u, causal = 0u;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const float4 t4 = *reinterpret_cast<const float4*>(&rs[64 + 8 * a4 + 4 * g]);
      const int ta[4] = {__float_as_int(t4.x), __float_as_int(t4.y), __float_as_int(t4.z), __float_as_int(t4.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rowok |= ta[e] >= 0 ? (1u << (4 * a4 + e)) : 0u;
        causal |= key <= ta[e] ? (1u << (4 * a4 + e)) : 0u;   // t = -1: no row
      }
    }

    // ---- role 0: S = Q K^T, role 1: dP = G_s V^T [32 q x 32 keys];
    // lane: key col, queries 8(i/4)+4g+(i%4)
    f32x16 x = f32x16{};
    {
      const uint16_t* A = role ? Fs : Qs;
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) x = mfma32x32x16(rdA(A, ds), kvb[ds], x);
    }
    // w: role 0 P, role 1 dS -- the B operand of the wave's product
    float w[16];
    if (role == 0) {
      // ---- P = 2^(S c - lse_s) on the causal keys -> LDS for role 1
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 l4 = *reinterpret_cast<const float4*>(&rs[8 * a4 + 4 * g]);
        const float la[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * a4 + e;
          const float v = fast_exp2(x[i] * scale_log2 - la[e]);
          w[i] = (causal >> i) & 1u ? v : 0.f;
        }
        *reinterpret_cast<float4*>(px + 256 * a4) = make_float4(w[4 * a4], w[4 * a4 + 1], w[4 * a4 + 2], w[4 * a4 + 3]);
      }
    }
    lds_barrier();                     // P of every key half visible
    if (role != 0) {
      // ---- dS = P (dP - D)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 p4 = *reinterpret_cast<const float4*>(px + 256 * a4);
        const float4 d4 = *reinterpret_cast<const float4*>(&rs[32 + 8 * a4 + 4 * g]);
        w[4 * a4] = p4.x * (x[4 * a4] - d4.x);
        w[4 * a4 + 1] = p4.y * (x[4 * a4 + 1] - d4.y);
        w[4 * a4 + 2] = p4.z * (x[4 * a4 + 2] - d4.z);
        w[4 * a4 + 3] = p4.w * (x[4 * a4 + 3] - d4.w);
      }
      // ---- dS^T -> LDS (bf16): the dS rows, or the dQ reduction over the block's keys
      {
        const int r = 32 * kh + cx;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          uint2 u = make_uint2(pack_bf16x2(w[4 * a4], w[4 * a4 + 1]), pack_bf16x2(w[4 * a4 + 2], w[4 * a4 + 3]));
          *reinterpret_cast<uint2*>(&DS[r * 32 + 8 * swz_s(r, a4) + 4 * g]) = u;
        }
      }
      if constexpr (DSOUT) {
        // ---- the rows of dS of this wave's 32 keys -> HBM for the query-
        // stationary dQ: the transposes of the wave's own dS^T rows for k-step
        // ks = 2 kh + h give lane (query col, g) element s = key 16 ks +
        // 8 (s / 4) + 4 g + s % 4.  A row of 32 keys is stored in the dQ
        // kernel's lane order, position 16 g' + 4 a + e for key 8 a + 4 g' + e,
        // so that element s of half h goes to position 16 g + 8 h + s.
        // (the transposes take all lanes, outside the store's lane condition:
        // a lane's result holds other lanes' reads)
        uint4 u[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) u[h] = __builtin_bit_cast(uint4, rdS(2 * kh + h));
        const int idx = it * 32 + col;
        if (idx < n) {
          uint16_t* dst = a.ds_rows + static_cast<int64_t>(p0 + idx) * kBlk + 32 * kh;
#pragma unroll
          for (int h = 0; h < 2; ++h) *reinterpret_cast<uint4*>(dst + 16 * g + 8 * h) = u[h];
        }
      }
    }
    // ---- role 0: dV^T += G_s^T P, role 1: dK^T += Q^T dS  (k = queries; 2 steps of 16)
    {
      const uint16_t* T = role ? Qs : Fs;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int o = 8 * st;
        const bf16x8 bw = to_bf16x8(w[o], w[o + 1], w[o + 2], w[o + 3], w[o + 4], w[o + 5], w[o + 6], w[o + 7]);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32x32x16(rdT(T, st, dt), bw, acc[dt]);
      }
    }
    if (more) {
      hold_sources();
      store_rows(Rn, ok_next);
      store_tiles(Qn, Fn);
    }
    if constexpr (DSOUT) {
      __builtin_amdgcn_s_waitcnt(0);   // the next batch's copies landed
      __syncthreads();
    } else {
      lds_barrier();                   // the next batch's tiles and dS^T in LDS
    }

    // ---- dQ[32 q x slice] of the batch = dS[32 q x block keys] K[block keys x slice]
    if (!DSOUT && has_slice) {
      f32x16 dq[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) dq[dt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2 * KH; ++ks) {
        const bf16x8 ds_op = rdS(ks);
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) dq[dt] = mfma32x32x16(ds_op, kq[ks][dt], dq[dt]);
      }
      // the batch's entries are p0 + 32 it + r (r: the query of register i)
      const int64_t e0 = static_cast<int64_t>(p0) + it * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!((rowok >> i) & 1u)) continue;
        const int r = 8 * (i >> 2) + 4 * g + (i & 3);
        uint16_t* dst = a.dq_part + (e0 + r) * kD + kSlice * wave + col;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) dst[32 * dt] = to_bf16(scale * dq[dt][i]).bits;
      }
    }
  };

  // prologue: the first batch
  load_rows(entry(0), live(0));
  load_tiles(entry(0), live(0), Q0, F0);
  store_rows(R0, live(0));
  store_tiles(Q0, F0);
  int e_next = entry(1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (DSOUT) {
    for (int it = 0; it < nbat; it += 2) {
      int e_after = entry(it + 2);
      step(it, e_next, Q0, F0, R0, Q1, F1, R1);
      e_next = e_after;
      if (it + 1 >= nbat) break;
      e_after = entry(it + 3);
      step(it + 1, e_next, Q1, F1, R1, Q0, F0, R0);
      e_next = e_after;
    }
  } else {
    for (int it = 0; it < nbat; ++it) {
      const int e_after = entry(it + 2);
      const bool odd = it & 1;
      step(it, e_next, odd ? Q1 : Q0, odd ? F1 : F0, odd ? R1 : R0, odd ? Q0 : Q1, odd ? F0 : F1, odd ? R0 : R1);
      e_next = e_after;
    }
  }
  write_out(acc);
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
    // every slot's partial loads at once (an absent slot loads entry 0, a
    // real address, and its contribution is selected away), then the sums
    // in slot order
    const int nslot = min(LR, Kc - e0);
    uint4 u[LR];
    bool ok[LR];
#pragma unroll
    for (int i = 0; i < LR; ++i) {
      ok[i] = i < nslot && __shfl(j, i, LR) >= 0;
      const uint32_t plo = __shfl(static_cast<uint32_t>(p), i, LR);
      const uint32_t phi = __shfl(static_cast<uint32_t>(p >> 32), i, LR);
      const int64_t pi = ok[i] ? (static_cast<int64_t>(phi) << 32) | plo : 0;
      u[i] = *reinterpret_cast<const uint4*>(part + pi * kD + 8 * li);
    }
#pragma unroll
    for (int i = 0; i < LR; ++i) {
      const uint32_t wd[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        acc[2 * k2] += ok[i] ? __uint_as_float(wd[k2] << 16) : 0.f;
        acc[2 * k2 + 1] += ok[i] ? __uint_as_float(wd[k2] & 0xffff0000u) : 0.f;
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
  auto go = [&](auto kern, int kh) {       // 2 kh waves: (key half, role)
    hipLaunchKernelGGL(kern, grid, dim3(128 * kh), 0, s, a, D.Hq, D.G, D.N, D.nb, D.scale, scale_log2);
  };
  const bool rows_out = a.ds_rows != nullptr;
  auto by_block = [&](auto hd_tag) {
    constexpr int HD = decltype(hd_tag)::value;
    if (D.block == 32) rows_out ? go(k_bwd_sparse<1, true, HD>, 1) : go(k_bwd_sparse<1, false, HD>, 1);
    else if (D.block == 64) rows_out ? go(k_bwd_sparse<2, true, HD>, 2) : go(k_bwd_sparse<2, false, HD>, 2);
    else rows_out ? go(k_bwd_sparse<4, true, HD>, 4) : go(k_bwd_sparse<4, false, HD>, 4);
  };
  if (D.d == 64) by_block(std::integral_constant<int, 64>{});
  else by_block(std::integral_constant<int, 128>{});
  timing_end(kKBwdSparse, s);
}

}  // namespace ssa
