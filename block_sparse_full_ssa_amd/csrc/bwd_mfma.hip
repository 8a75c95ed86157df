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
//   bwd_pre:  per row, G_f / G_s in bf16, D_f / D_s from the rounded G, the
//             lse values in log2 units, and (sparse stream alone) a zeroed
//             fp32 dQ accumulator row;
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

constexpr int kD = 128;
constexpr int kBN = 128;       // keys per workgroup
constexpr int kBM = 32;        // queries per iteration
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bwd_pre --
__global__ void __launch_bounds__(256)
    k_bwd_pre(BwdPreArgs a, int64_t rows, float w_f, float w_s_align, float inv_m) {
  // 16 lanes per row, 8 elements (16 bytes) each; 16 rows per workgroup
  const int li = threadIdx.x & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
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
  for (int o = 8; o >= 1; o >>= 1) {
    Df += __shfl_xor(Df, o, 16);
    Ds += __shfl_xor(Ds, o, 16);
  }
  if (!ok) return;
  if (has_f) *reinterpret_cast<uint4*>(a.g_full + off) = make_uint4(gfw[0], gfw[1], gfw[2], gfw[3]);
  if (has_s) *reinterpret_cast<uint4*>(a.g_sparse + off) = make_uint4(gsw[0], gsw[1], gsw[2], gsw[3]);
  if (a.dq_acc) {
    *reinterpret_cast<float4*>(a.dq_acc + off) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(a.dq_acc + off + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (li == 0) {
    if (has_f) {
      a.D_full[row] = Df;
      a.lse2_full[row] = a.lse_full[row] * kLog2e;
    }
    if (has_s) {
      a.D_sparse[row] = Ds;
      a.lse2_sparse[row] = a.lse_sparse[row] * kLog2e;
    }
  }
}

// --------------------------------------------------------------- bwd_mfma --
// Physical 16-byte chunk of logical chunk c in a 256-byte Q / G row r (read by
// rows and by transposes).
// The transposed tiles use c ^ (2 (r % 8) + (r / 8) % 2): measured on gfx950
// it keeps the transpose reads (ds_read_b64_tr_b16) free of bank conflicts
// as well as the 16-byte row reads, where c ^ (r % 8) or c ^ (r % 16) leave
// the transpose reads two-way conflicted.
__device__ __forceinline__ int swz_t(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__global__ void __launch_bounds__(256, 2)
    k_bwd_mfma(BwdMainArgs a, int Hq, int G, int N, float scale, float scale_log2) {
  // Two workgroups per CU, so that the two waves on a SIMD belong to
  // different workgroups and drift apart: one's waits (LDS, the softmax, the
  // barrier) overlap the other's MFMAs.  A workgroup owns 128 keys (32 per
  // wave); K of the 128 keys sits in LDS as an MFMA operand, V in registers.
  // LDS: K (32 KiB) and two sets of {Q, G_f tiles [32][128], row values}.
  constexpr int kT = kBM * kD;                       // one Q / G tile
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kBN * kD];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[kT], F0[kT], Q1[kT], F1[kT];
  __shared__ __attribute__((aligned(16))) float R0[2 * kBM], R1[2 * kBM];

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

  // K of the 128 keys -> LDS: 32 instructions of 1 KiB (4 rows), 8 per wave;
  // lane l fills physical chunk l % 16 of row 4n + l / 16 with the logical
  // chunk stored there; keys past N repeat the last key (their pairs are masked)
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int n = wave * 8 + r;                     // uniform
    const int row = 4 * n + (lane >> 4);
    const int64_t key = min(k0 + row, N - 1);
    __builtin_amdgcn_global_load_lds((const glb_void*)(kg + key * kD + 8 * swz_t(row, lane & 15)),
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
  // Q / G_f tiles of one iteration: 16 instructions, 4 per wave; the tile
  // bases are uniform, the lane offsets fixed
  // (byte offsets, so that each load is a scalar base plus a 32-bit lane offset)
  uint32_t dmo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * ((wave * 4 + r) & 7) + (lane >> 4);
    dmo[r] = 2 * (row * kD + 8 * swz_t(row, lane & 15));
  }
  auto load_tiles = [&](int hq, int q0, uint16_t* Qd, uint16_t* Fd) {
    const int64_t tile = ((static_cast<int64_t>(b) * Hq + hq) * N + q0) * (kD * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = wave * 4 + r;                   // 0..15, uniform
      const char* src = static_cast<const char*>((n >> 3) ? a.g_full : a.q) + tile;
      uint16_t* dst = (n >> 3) ? Fd : Qd;
      __builtin_amdgcn_global_load_lds((const glb_void*)(src + dmo[r]), (lds_void*)(dst + (n & 7) * 512), 16, 0, 0);
    }
  };
  // row values (lse2, D) through registers
  float prow = 0.f;
  auto load_rows = [&](int hq, int q0) {
    const int64_t rowbase = (static_cast<int64_t>(b) * Hq + hq) * N + q0;
    if (wave == 0) {                      // lanes 0-31: lse2 of the 32 rows, 32-63: D
      if (lane < kBM) prow = a.lse2_full[rowbase + lane];
      else prow = a.D_full[rowbase + lane - kBM];
    }
  };

  f32x16 dv[4], dk[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dv[dt] = f32x16{};
    dk[dt] = f32x16{};
  }

  // one iteration on set (Qs, Fs, rv) while the next streams into (Qn, Fn, Rn)
  auto step = [&](int it, int q0, int hq1, int q01, const uint16_t* Qs, const uint16_t* Fs, const float* rv,
                  uint16_t* Qn, uint16_t* Fn, float* Rn) {
    const bool more = it + 1 < iters;
    if (more) {
      load_rows(hq1, q01);    // plain loads first: no VMEM load may follow the copies
      load_tiles(hq1, q01, Qn, Fn);
    }
    const bool wave_has_pairs = q0 + kBM - 1 >= kw0 && kw0 < N;   // uniform
    const bool diag = q0 < kw0 + 31;                               // some key > some query

    if (wave_has_pairs) {
      // LDS offsets, rebuilt from lane constants in every iteration.  Row
      // reads of d-step ds: base + 16 (ds ^ (col % 8)); transpose reads of
      // (st, dt): tb + 2048 st + 32 (dt ^ tx), the second row eight below at tb1
      int c7 = col & 7, tx = 2 * gk + (srow >> 1);
      asm volatile("" : "+v"(c7), "+v"(tx));
      const int rowq = col * kD + 8 * (g ^ ((col >> 3) & 1));
      const int rowk = (32 * kq + col) * kD + 8 * (g ^ ((col >> 3) & 1));
      const int tb0 = (4 * gk + srow) * kD + 8 * ((2 * (grp & 1) + (m4 >> 1)) ^ (2 * (srow & 1))) + 4 * (m4 & 1);
      const int tb1 = tb0 + 8 * kD + 8 * (1 - 2 * ((m4 >> 1) & 1));
      // ---- S = Q K^T, dP = G_f V^T  [32 q x 32 keys], two independent
      // accumulation chains interleaved, operands read one step ahead; lane:
      // key col, queries 8(i/4)+4g+(i%4)
      f32x16 s = f32x16{}, dpf = f32x16{};
      bf16x8 ok[8], oq[8], of[8];
      auto rd = [&](int ds) {
        const int cs = 16 * (ds ^ c7);   // the same chunk for query row col and key row 32 kq + col
        ok[ds] = lds_read8(&Kt[rowk + cs]);
        oq[ds] = lds_read8(&Qs[rowq + cs]);
        of[ds] = lds_read8(&Fs[rowq + cs]);
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
      // ---- probabilities and dS, packed to bf16 pairs (register i: query
      // 8(i/4) + 4g + i%4, visible iff 8(i/4) + i%4 >= t on diagonal tiles;
      // dS of a masked pair is zero because its P is)
      float p[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 lf = *reinterpret_cast<const float4*>(&rv[8 * a4 + 4 * g]);
        const float lfa[4] = {lf.x, lf.y, lf.z, lf.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) p[4 * a4 + k] = fast_exp2(s[4 * a4 + k] * scale_log2 - lfa[k]);
      }
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
        const float4 df = *reinterpret_cast<const float4*>(&rv[kBM + 8 * a4 + 4 * g]);
        const float dfa[4] = {df.x, df.y, df.z, df.w};
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = p[4 * a4 + k] * (dpf[4 * a4 + k] - dfa[k]);
        pfp[2 * a4] = pack_bf16x2(p[4 * a4], p[4 * a4 + 1]);
        pfp[2 * a4 + 1] = pack_bf16x2(p[4 * a4 + 2], p[4 * a4 + 3]);
        dsp[2 * a4] = pack_bf16x2(e[0], e[1]);
        dsp[2 * a4 + 1] = pack_bf16x2(e[2], e[3]);
      }
      // ---- dV^T += G^T P, dK^T += Q^T dS  (k = queries; 2 steps of 16),
      // transpose reads one step ahead
      bf16x8 bpf[2], bds[2], tg[8], tq[8];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bpf[st] = __builtin_bit_cast(bf16x8, make_uint4(pfp[4 * st], pfp[4 * st + 1], pfp[4 * st + 2], pfp[4 * st + 3]));
        bds[st] = __builtin_bit_cast(bf16x8, make_uint4(dsp[4 * st], dsp[4 * st + 1], dsp[4 * st + 2], dsp[4 * st + 3]));
      }
      auto rdB = [&](int u) {
        const int cx = 2048 * (u >> 2) + 32 * ((u & 3) ^ tx);
        tg[u] = lds_tr_pair(&Fs[tb0 + cx], &Fs[tb1 + cx]);
        tq[u] = lds_tr_pair(&Qs[tb0 + cx], &Qs[tb1 + cx]);
      };
      rdB(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < 8) rdB(u + 1);
        dv[u & 3] = mfma32x32x16(tg[u], bpf[u >> 2], dv[u & 3]);
        dk[u & 3] = mfma32x32x16(tq[u], bds[u >> 2], dk[u & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more && tid < 2 * kBM) Rn[tid] = prow;
    __builtin_amdgcn_s_waitcnt(0);     // next tiles landed
    __syncthreads();
  };

  int hq = c * G, q0 = N - kBM;                    // iteration it
  int hq1 = hq, q01 = q0;                           // iteration it + 1
  advance(hq1, q01);
  load_rows(hq, q0);
  load_tiles(hq, q0, Q0, F0);
  if (tid < 2 * kBM) R0[tid] = prow;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < iters; it += 2) {
    step(it, q0, hq1, q01, Q0, F0, R0, Q1, F1, R1);
    q0 = q01;
    advance(hq1, q01);
    if (it + 1 >= iters) break;
    step(it + 1, q0, hq1, q01, Q1, F1, R1, Q0, F0, R0);
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
    for (int dt = 0; dt < 4; ++dt) {
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

bool bwd_mfma_supported(const Dims& D) { return D.dtype == 1 && D.d == kD; }

void launch_bwd_pre(const Dims& D, const BwdPreArgs& a, float w_sparsity, float w_commit, hipStream_t s) {
  const float inv_m = static_cast<float>(1.0 / static_cast<double>(D.q_elems()));
  dim3 grid(static_cast<unsigned>((D.rows() + 15) / 16));
  timing_begin(kKBwdPre, s);
  hipLaunchKernelGGL(k_bwd_pre, grid, dim3(256), 0, s, a, D.rows(), w_sparsity, w_commit, inv_m);
  timing_end(kKBwdPre, s);
}

void launch_bwd_mfma(const Dims& D, const BwdMainArgs& a, hipStream_t s) {
  dim3 grid(D.B * D.Hkv, (D.N + kBN - 1) / kBN);
  timing_begin(kKBwdMfma, s);
  hipLaunchKernelGGL(k_bwd_mfma, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.scale, D.scale * kLog2e);
  timing_end(kKBwdMfma, s);
}

}  // namespace ssa
