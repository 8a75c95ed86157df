// Backward of SSA dual-stream attention, bf16 MFMA on gfx950: the stream
// gradients and the full stream.
//
// Each output receives its own gradient (Sintesi Tecnica, section 2,
// 'Allineamento Bidirezionale'): the upstream gradient goes to the active
// stream only, L_sparsity adds (2/M) w_s (h_full - h_sparse) to the full
// stream and L_commit adds (2/M) w_c (h_sparse - h_full) to the sparse
// stream (the other output held fixed in each).  With those stream
// gradients G_f, G_s the two streams are differentiated separately and the
// results added: the sparse stream on key-block buckets (sparse_bwd.hip),
// the full stream here:
//   P   = 2^(S c - lse_f)                          (c = scale * log2 e)
//   dS  = P (G_f V^T - D_f),  D_f = rowsum(G_f o h_full)
//   dV  = P^T G_f,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Kernels:
//   bwd_pre:  per row, G_f / G_s in bf16, D_f / D_s from the rounded G and
//             the lse values in log2 units;
//   bwd_mfma: dK / dV, key-stationary.  A workgroup owns 128 keys of one KV
//             head (32 per wave; K in LDS, V in registers as MFMA operands)
//             and walks the G query heads of the group and every 32-query
//             tile at or after its keys.  Two workgroups share a CU, so the
//             two waves on a SIMD come from different workgroups and overlap
//             each other's waits.  dK and dV accumulate in registers over
//             all tiles (no atomics) and leave with the sparse stream's fp32
//             dK / dV added;
//   bwd_dq:   dQ of both streams, query-stationary (bwd_dq.hip).
//
// Layout: the logits are kept as S = Q K^T (lane l owns key l % 32 and 16
// queries), which is the B-operand layout of dV^T = G^T P and dK^T = Q^T dS;
// the transposed A operands G^T and Q^T come from row-major LDS tiles
// through transpose reads.  All MFMA guards are wave-uniform.

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kBN = 128;       // keys per workgroup
constexpr int kBM = 32;        // queries per iteration
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bwd_pre --
template <int HD>   // head dimension
__global__ void __launch_bounds__(256)
    k_bwd_pre(BwdPreArgs a, int64_t rows, float w_f, float w_s_align, float inv_m, float scale_log2) {
  // LR = HD / 8 lanes per row, 8 elements (16 bytes) each; 256 / LR rows per workgroup
  constexpr int kD = HD, LR = HD / 8;
  const int li = threadIdx.x % LR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / LR) + (threadIdx.x / LR);
  const bool ok = row < rows;
  const int64_t off = (ok ? row : 0) * kD + 8 * li;
  const bool has_f = a.mode != kSparseOnly, has_s = a.mode != kFullOnly;
  const bool dual = a.mode == kDualFull || a.mode == kDualSparse;
  const bool up_f = a.mode == kDualFull || a.mode == kFullOnly;
  auto load8 = [&](const void* p, float* x) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (p && ok) u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  };
  float g[8], vf[8], vs[8];
  load8(a.dout, g);
  load8(has_f ? a.h_full : nullptr, vf);
  load8(has_s ? a.h_sparse : nullptr, vs);
  float Df = 0.f, Ds = 0.f;
  uint32_t gfw[4], gsw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float gf2[2], gs2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * k + e;
      float gf = 0.f, gs = 0.f;
      if (dual) {
        const float diff = vf[i] - vs[i];
        gf = w_f * 2.f * inv_m * diff + (up_f ? g[i] : 0.f);
        gs = -w_s_align * 2.f * inv_m * diff + (up_f ? 0.f : g[i]);
      } else {
        gf = up_f ? g[i] : 0.f;
        gs = up_f ? 0.f : g[i];
      }
      gf2[e] = to_f32(to_bf16(gf));            // the stored (rounded) gradients
      gs2[e] = to_f32(to_bf16(gs));
      Df += gf2[e] * vf[i];
      Ds += gs2[e] * vs[i];
    }
    gfw[k] = pack_bf16x2(gf2[0], gf2[1]);
    gsw[k] = pack_bf16x2(gs2[0], gs2[1]);
  }
#pragma unroll
  for (int o = LR / 2; o >= 1; o >>= 1) {
    Df += __shfl_xor(Df, o, LR);
    Ds += __shfl_xor(Ds, o, LR);
  }
  if (!ok) return;
  if (has_f) *reinterpret_cast<uint4*>(a.g_full + off) = make_uint4(gfw[0], gfw[1], gfw[2], gfw[3]);
  if (has_s) *reinterpret_cast<uint4*>(a.g_sparse + off) = make_uint4(gsw[0], gsw[1], gsw[2], gsw[3]);
  if (li == 0) {
    if (has_f) {
      const float l2 = a.lse_full[row] * kLog2e;
      a.D_full[row] = Df;
      a.lse2_full[row] = l2;
      const uint2 tl = split3_bf16(-l2 * (1.f / scale_log2)), td = split3_bf16(-Df);
      a.rowv_full[row] = make_uint4(tl.x, tl.y, td.x, td.y);
    }
    if (has_s) {
      a.D_sparse[row] = Ds;
      a.lse2_sparse[row] = a.lse_sparse[row] * kLog2e;
    }
  }
}

// --------------------------------------------------------------- bwd_mfma --
// Physical 16-byte chunk of logical chunk c in a K / Q / G row r of 2 HD bytes
// (read by rows and by transposes): swz256 for 256-byte rows (HD = 128),
// swz128 for 128-byte rows (HD = 64).
template <int HD> __device__ __forceinline__ int swz_t(int r, int c) {
  return HD == 128 ? swz256(r, c) : swz128(r, c);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

template <int HD>   // head dimension
__global__ void __launch_bounds__(256, 2)
    k_bwd_mfma(BwdMainArgs a, int Hq, int G, int N, float scale, float scale_log2) {
  // Two workgroups per CU, so that the waves on a SIMD belong to different
  // workgroups and drift apart: one's waits (LDS, the softmax, the barrier)
  // overlap the other's MFMAs (three spill at HD = 64).  A workgroup owns 128
  // keys (32 per wave); K of the 128 keys sits in LDS as an MFMA operand, V
  // in registers.  LDS: K (32 KiB at HD = 128) and two sets of {Q, G_f tiles
  // [32][HD]}.
  constexpr int kD = HD;
  constexpr int kDT = HD / 32;                       // 32-column tiles of dK / dV
  constexpr int kCh = HD / 8;                        // 16-byte chunks per row
  constexpr int kRowsOp = 512 / HD;                  // rows of one 1 KiB copy
  constexpr int kT = kBM * kD;                       // one Q / G tile
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kBN * kD];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[kT], F0[kT], Q1[kT], F1[kT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, li = lane & 15;
  const int gk = grp >> 1, srow = li >> 2, m4 = li & 3;

  const int bc = blockIdx.x;                        // batch * Hkv + kv head
  const int Hkv = Hq / G;
  // the division runs on the vector unit: bring the results back to scalars
  const int b = __builtin_amdgcn_readfirstlane(bc / Hkv);
  const int c = bc - b * Hkv;
  const int k0 = blockIdx.y * kBN;
  const int kw0 = k0 + 32 * kq;                     // this wave's first key
  const int64_t kvbase = static_cast<int64_t>(bc) * N * kD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + kvbase;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + kvbase;

  // N is a multiple of 32 (block >= 32 divides it), so query tiles are whole.
  const int nqt = N / kBM;
  const int qt0 = k0 / kBM;                         // first query tile that sees these keys
  const int iters = G * (nqt - qt0);                // >= G >= 1

  // K of the 128 keys -> LDS: instructions of 1 KiB (kRowsOp rows), a quarter
  // per wave; lane l fills physical chunk l % kCh of row kRowsOp n + l / kCh
  // with the logical chunk stored there; keys past N repeat the last key
  // (their pairs are masked)
  constexpr int kOpsK = kBN / kRowsOp / 4;
#pragma unroll
  for (int r = 0; r < kOpsK; ++r) {
    const int n = wave * kOpsK + r;                 // uniform
    const int row = kRowsOp * n + lane / kCh;
    const int64_t key = min(k0 + row, N - 1);
    __builtin_amdgcn_global_load_lds((const glb_void*)(kg + key * kD + 8 * swz_t<HD>(row, lane % kCh)),
                                     (lds_void*)(Kt + n * 512), 16, 0, 0);
  }
  // dP B operand [16 d x 32 keys] from registers: key = kw0 + col, d = 16 ds + 8 g + s
  bf16x8 vb[kD / 16];
  {
    const int key = kw0 + col;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (key < N) w = *reinterpret_cast<const uint4*>(vg + static_cast<int64_t>(key) * kD + 16 * ds + 8 * g);
      vb[ds] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // iteration coordinates (query head, first query), advanced incrementally:
  // the group's heads inner, query tiles from the last one down to the first
  // that sees these keys.  The workgroups of a KV head that start together
  // then read the same Q / G_f tile at about the same time, so one L2 fill
  // serves them all (ascending tiles put them 4 tiles apart, and heads outer
  // lets them drift onto different heads).
  auto advance = [&](int& hq, int& q0) {
    if (++hq == (c + 1) * G) {
      hq = c * G;
      q0 -= kBM;
    }
  };
  // Q / G_f tiles of one iteration: HD / 16 instructions of 1 KiB per tile,
  // HD / 32 per wave; the tile bases are uniform, the lane offsets fixed
  // (byte offsets, so that each load is a scalar base plus a 32-bit lane offset)
  constexpr int kOpsT = HD / 16, kOpsW = HD / 32;
  uint32_t dmo[kOpsW];
#pragma unroll
  for (int r = 0; r < kOpsW; ++r) {
    const int row = kRowsOp * ((wave * kOpsW + r) % kOpsT) + lane / kCh;
    dmo[r] = 2 * (row * kD + 8 * swz_t<HD>(row, lane % kCh));
  }
  auto load_tiles = [&](int hq, int q0, uint16_t* Qd, uint16_t* Fd) {
    const int64_t tile = ((static_cast<int64_t>(b) * Hq + hq) * N + q0) * kD;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(static_cast<const uint16_t*>(a.q) + tile, kT * 2);
    const __amdgpu_buffer_rsrc_t rg = tile_rsrc(a.g_full + tile, kT * 2);
#pragma unroll
    for (int r = 0; r < kOpsW; ++r) {
      const int n = wave * kOpsW + r;               // uniform
      const bool gt = n >= kOpsT;                   // the G tile's half of the copies
      buffer_to_lds16(gt ? rg : rq, (gt ? Fd : Qd) + (n % kOpsT) * 512, dmo[r]);
    }
  };
  // Row values of the 32 queries: lane l holds those of query l % 32.  They
  // enter the logits and dP through the accumulators: one extra matrix
  // product each starts S at -lse2 / c and dP at -D (A: the value's three
  // bf16 terms, written by bwd_pre, in the k-slots 0..2; B: ones in the same
  // slots of the lanes of k-group 0 and zeros elsewhere, so the k-group 1
  // lanes' copies of the terms add nothing), so no per-element row value has
  // to be fetched for the softmax and dS.
  u32x4 rv = u32x4{0u, 0u, 0u, 0u}, rv_n = rv;
  auto load_rows = [&](int hq, int q0) {
    const int64_t r = (static_cast<int64_t>(b) * Hq + hq) * N + q0 + col;
    rv_n = *reinterpret_cast<const u32x4*>(a.rowv_full + r);
  };
  const bf16x8 ones = __builtin_bit_cast(bf16x8, g ? make_uint4(0u, 0u, 0u, 0u)
                                                   : make_uint4(0x3F803F80u, 0x00003F80u, 0u, 0u));

  f32x16 dv[kDT], dk[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dv[dt] = f32x16{};
    dk[dt] = f32x16{};
  }
  // Byte offsets of the row reads of d-step ds: the same chunk of query row
  // col in the Q / G_f tiles and of key row 32 kq + col in K (the same
  // swizzle: rows 16 apart share it).  Those of the first half of the
  // d-steps are computed once and held in registers; d-step ds + kRO flips
  // one bit of d-step ds's (its logical chunk 2 ds + g flips the top bit,
  // and so does the physical one: bit 7 of the offset at HD = 128, bit 6 at
  // HD = 64), and the key row's adds kq_off, whose bits the query offsets
  // (< 64 HD) never use, so an OR.
  constexpr int kRO = kD / 32, kFlip = kD;
  int roff[kRO];
#pragma unroll
  for (int ds = 0; ds < kRO; ++ds)
    roff[ds] = 2 * (col * kD + 8 * swz_t<HD>(col, 2 * ds + g));
  const int kq_off = 2 * 32 * kq * kD;              // uniform
  auto qoff = [&](int ds) { return ds < kRO ? roff[ds] : roff[ds - kRO] ^ kFlip; };
  auto koff = [&](int ds) { return qoff(ds) | kq_off; };
  // Byte offsets of the transpose reads: those of k-step st and column tile
  // dt are trb[0] ^ 64 dt and trb[1] ^ 64 dt (rows eight apart) plus
  // 32 HD st.  The lane reads logical chunk 4 dt + y (y = 2 (grp % 2) +
  // m4 / 2) of row r = 16 st + 4 gk + srow (+ 8).  Its swizzle term is
  // 4 srow + gk (+ 2) at HD = 128 and 4 sb + gk (+ 2), sb = (srow / 2) % 2, at
  // HD = 64, so the physical chunk is 4 (dt ^ t) + (y ^ (gk (+ 2))) with t =
  // srow or sb, and in elements 32 (dt ^ t) = 32 t ^ 32 dt on the bits above
  // the chunk's low two, which the rest of the offset leaves clear.
  int trb[2];
  {
    const int y = 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
    const int t = HD == 128 ? srow : (srow >> 1) & 1;
    trb[0] = 2 * ((4 * gk + srow) * kD + 8 * (y ^ gk) + e4 + 32 * t);
    trb[1] = 2 * ((4 * gk + srow + 8) * kD + 8 * (y ^ (gk + 2)) + e4 + 32 * t);
  }
  auto tr16 = [](const uint16_t* base, int o0, int o1) {
    const char* b8 = reinterpret_cast<const char*>(base);
    return lds_tr_pair(reinterpret_cast<const uint16_t*>(b8 + o0), reinterpret_cast<const uint16_t*>(b8 + o1));
  };
  auto rd16 = [](const uint16_t* base, int off) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off));
  };

  // one iteration on set (Qs, Fs) while the next streams into (Qn, Fn)
  auto step = [&](int it, int q0, int hq1, int q01, const uint16_t* Qs, const uint16_t* Fs, uint16_t* Qn,
                  uint16_t* Fn) {
    const bool more = it + 1 < iters;
    rv = rv_n;
    if (more) {
      load_rows(hq1, q01);    // plain loads first: no VMEM load may follow the copies
      load_tiles(hq1, q01, Qn, Fn);
    }
    const bool wave_has_pairs = q0 + kBM - 1 >= kw0 && kw0 < N;   // uniform
    const bool diag = q0 < kw0 + 31;                               // some key > some query

    if (wave_has_pairs) {
      // ---- S = Q K^T, dP = G_f V^T  [32 q x 32 keys], two independent
      // accumulation chains interleaved, operands read one step ahead; lane:
      // key col, queries 8(i/4)+4g+(i%4)
      f32x16 s = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{rv[0], rv[1], 0u, 0u}), ones, f32x16{});
      f32x16 dpf = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{rv[2], rv[3], 0u, 0u}), ones, f32x16{});
      bf16x8 ok[8], oq[8], of[8];
      // (opaque to the compiler, so that the derived offsets are rebuilt
      // here rather than hoisted out of the loop into more registers)
#pragma unroll
      for (int i = 0; i < kRO; ++i) asm volatile("" : "+v"(roff[i]));
      asm volatile("" : "+v"(trb[0]), "+v"(trb[1]));
      auto rd = [&](int ds) {
        const int o = qoff(ds);
        ok[ds] = rd16(Kt, koff(ds));
        oq[ds] = rd16(Qs, o);
        of[ds] = rd16(Fs, o);
      };
      rd(0);
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) {
        __builtin_amdgcn_sched_barrier(0);
        if (ds + 1 < kD / 16) rd(ds + 1);
        s = mfma32x32x16(oq[ds], ok[ds], s);
        dpf = mfma32x32x16(of[ds], vb[ds], dpf);
      }
      __builtin_amdgcn_sched_barrier(0);
      // G^T and Q^T operands of the dV / dK products (step u: k-step u / kDT
      // of 16 queries, column tile u % kDT), read two steps ahead: the first
      // two during the softmax
      bf16x8 tg[2 * kDT], tq[2 * kDT];
      auto rdB = [&](int u) {
        const int x0 = (trb[0] ^ (64 * (u % kDT))) + 32 * kD * (u / kDT);
        const int x1 = (trb[1] ^ (64 * (u % kDT))) + 32 * kD * (u / kDT);
        tg[u] = tr16(Fs, x0, x1);
        tq[u] = tr16(Qs, x0, x1);
      };
      rdB(0);
      rdB(1);
      __builtin_amdgcn_sched_barrier(0);
      // ---- probabilities and dS, packed to bf16 pairs (register i: query
      // 8(i/4) + 4g + i%4, visible iff 8(i/4) + i%4 >= t on diagonal tiles;
      // dS of a masked pair is zero because its P is)
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i] * scale_log2);
      if (diag) {
        // uniform, and taken on one tile per wave and head, so a real branch
        // (the empty asm keeps the compiler from turning it into selects)
        asm volatile("");
        const int t = kw0 + col - q0 - 4 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = 8 * (i / 4) + i % 4 >= t ? p[i] : 0.f;
      }
      uint32_t pfp[8], dsp[8];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = p[4 * a4 + k] * dpf[4 * a4 + k];
        pfp[2 * a4] = pack_bf16x2(p[4 * a4], p[4 * a4 + 1]);
        pfp[2 * a4 + 1] = pack_bf16x2(p[4 * a4 + 2], p[4 * a4 + 3]);
        dsp[2 * a4] = pack_bf16x2(e[0], e[1]);
        dsp[2 * a4 + 1] = pack_bf16x2(e[2], e[3]);
      }
      // ---- dV^T += G^T P, dK^T += Q^T dS  (k = queries; 2 steps of 16)
      bf16x8 bpf[2], bds[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bpf[st] = __builtin_bit_cast(bf16x8, make_uint4(pfp[4 * st], pfp[4 * st + 1], pfp[4 * st + 2], pfp[4 * st + 3]));
        bds[st] = __builtin_bit_cast(bf16x8, make_uint4(dsp[4 * st], dsp[4 * st + 1], dsp[4 * st + 2], dsp[4 * st + 3]));
      }
#pragma unroll
      for (int u = 0; u < 2 * kDT; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (u + 2 < 2 * kDT) {
          rdB(u + 2);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // the reads, then the products
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        dv[u % kDT] = mfma32x32x16(tg[u], bpf[u / kDT], dv[u % kDT]);
        dk[u % kDT] = mfma32x32x16(tq[u], bds[u / kDT], dk[u % kDT]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);     // next tiles landed
    __syncthreads();
  };

  int hq = c * G, q0 = N - kBM;                    // iteration it
  int hq1 = hq, q01 = q0;                           // iteration it + 1
  advance(hq1, q01);
  load_rows(hq, q0);
  load_tiles(hq, q0, Q0, F0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < iters; it += 2) {
    step(it, q0, hq1, q01, Q0, F0, Q1, F1);
    q0 = q01;
    advance(hq1, q01);
    if (it + 1 >= iters) break;
    step(it + 1, q0, hq1, q01, Q1, F1, Q0, F0);
    q0 = q01;
    advance(hq1, q01);
  }

  // ---- epilogue: dK = scale * dK^T^T (+ sparse stream), dV (+ sparse stream),
  // in bf16; lane owns key kw0 + col
  const int key = kw0 + col;
  if (key < N) {
    const int64_t kro = kvbase + static_cast<int64_t>(key) * kD;
    uint16_t* dkg = static_cast<uint16_t*>(a.dk) + kro;
    uint16_t* dvg = static_cast<uint16_t*>(a.dv) + kro;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * g;
        const int i = 4 * a4;
        float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xv = xk;
        if (a.dk_part) {
          xk = *reinterpret_cast<const float4*>(a.dk_part + kro + d0);
          xv = *reinterpret_cast<const float4*>(a.dv_part + kro + d0);
        }
        *reinterpret_cast<uint2*>(dkg + d0) =
            make_uint2(pack_bf16x2(scale * dk[dt][i] + xk.x, scale * dk[dt][i + 1] + xk.y),
                       pack_bf16x2(scale * dk[dt][i + 2] + xk.z, scale * dk[dt][i + 3] + xk.w));
        *reinterpret_cast<uint2*>(dvg + d0) =
            make_uint2(pack_bf16x2(dv[dt][i] + xv.x, dv[dt][i + 1] + xv.y),
                       pack_bf16x2(dv[dt][i + 2] + xv.z, dv[dt][i + 3] + xv.w));
      }
    }
  }
}

}  // namespace

bool bwd_mfma_supported(const Dims& D) { return D.dtype == 1 && (D.d == 128 || D.d == 64); }

void launch_bwd_pre(const Dims& D, const BwdPreArgs& a, float w_sparsity, float w_commit, hipStream_t s) {
  const float inv_m = static_cast<float>(1.0 / static_cast<double>(D.q_elems()));
  const int rows_wg = D.d == 64 ? 32 : 16;
  dim3 grid(static_cast<unsigned>((D.rows() + rows_wg - 1) / rows_wg));
  timing_begin(kKBwdPre, s);
  const float scale_log2 = D.scale * kLog2e;
  if (D.d == 64)
    hipLaunchKernelGGL(k_bwd_pre<64>, grid, dim3(256), 0, s, a, D.rows(), w_sparsity, w_commit, inv_m, scale_log2);
  else
    hipLaunchKernelGGL(k_bwd_pre<128>, grid, dim3(256), 0, s, a, D.rows(), w_sparsity, w_commit, inv_m, scale_log2);
  timing_end(kKBwdPre, s);
}

void launch_bwd_mfma(const Dims& D, const BwdMainArgs& a, hipStream_t s) {
  dim3 grid(D.B * D.Hkv, (D.N + kBN - 1) / kBN);
  timing_begin(kKBwdMfma, s);
  if (D.d == 64) hipLaunchKernelGGL(k_bwd_mfma<64>, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.scale, D.scale * kLog2e);
  else hipLaunchKernelGGL(k_bwd_mfma<128>, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.scale, D.scale * kLog2e);
  timing_end(kKBwdMfma, s);
}

}  // namespace ssa
