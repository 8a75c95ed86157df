// dQ of SSA's full stream, bf16 MFMA on gfx950, query-stationary.
//
// The full stream's query gradient (Sintesi Tecnica, section 2: the full
// output's stream gradient G_f through the causal softmax) is
//   dQ = scale sum over keys of P (G_f V^T - D_f) K,   P = 2^(S c - lse_f).
// A workgroup owns 128 queries of one head (32 per wave) and walks the
// causal key tiles of 64 keys, recomputing the logits and dP on the way, so
// that dQ accumulates in registers: no atomics and no exchange through LDS.
// The layout is the forward's: S^T = K Q^T and dP^T = V G^T (A = K / V rows
// from LDS, B = the wave's Q / G rows in registers) leave lane l with query
// l % 32; dS^T = P^T (dP^T - D) is then the B operand of dQ^T += K^T dS^T,
// with K^T read from the same K tile by transpose reads.  K / V tiles move
// HBM -> LDS double-buffered, one barrier per tile.
//
// Training modes add the sparse stream here as well: its dS rows (written by
// the bucketed sparse backward, bf16) for the wave's queries that selected a
// half's key block are added to the full stream's dS^T before the product,
// so both streams share one dQ^T accumulation and no atomics are needed.  A
// wave's 32 queries are one word of the block's bucket mask; a selected
// query's row is entry wpos + popcount of the word's lower bits.

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kD = 128;
constexpr int kBM = 128;         // queries per workgroup
constexpr int kBN = 64;          // keys per tile
constexpr int kTile = kBN * kD;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Physical 16-byte chunk of logical chunk c in a 256-byte K / V row r (K is
// read by rows and by transposes).
// The transposed tiles use c ^ (2 (r % 8) + (r / 8) % 2): measured on gfx950
// it keeps the transpose reads (ds_read_b64_tr_b16) free of bank conflicts
// as well as the 16-byte row reads, where c ^ (r % 8) or c ^ (r % 16) leave
// the transpose reads two-way conflicted.
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (((r & 7) << 1) | ((r >> 3) & 1)); }

template <bool SPARSE>
__global__ void __launch_bounds__(256, 2)
    k_bwd_dq(BwdDqArgs a, int Hq, int G, int N, int nb, int block, float scale, float scale_log2, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t K0[kTile], K1[kTile], V0[kTile], V1[kTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, li = lane & 15;
  const int gk = grp >> 1, srow = li >> 2, m4 = li & 3;
  const QTileItem item = qtile_item(blockIdx.x, static_cast<int>(gridDim.x) / (n_qtiles * G), G, n_qtiles);
  const int bh = item.bh;
  const int q0 = (n_qtiles - 1 - item.rank) * kBM;   // longest tiles first
  const int b = bh / Hq, h = bh % Hq;
  const int64_t bc = static_cast<int64_t>(b) * (Hq / G) + h / G;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + bc * N * kD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + bc * N * kD;

  const int qrow = q0 + wave * 32 + col;           // this lane's query
  const bool wave_live = q0 + wave * 32 < N;
  const int wave_q0 = q0 + wave * 32;
  const int wave_last_q = min(N - 1, wave_q0 + 31);
  const int64_t row = static_cast<int64_t>(bh) * N + qrow;
  // the wave's Q and G_f rows as B operands (query = col, d = 16 ds + 8 g + s)
  bf16x8 qreg[kD / 16], greg[kD / 16];
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) {
    uint4 u = make_uint4(0, 0, 0, 0), w = make_uint4(0, 0, 0, 0);
    if (qrow < N) {
      u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + row * kD + 16 * ds + 8 * g);
      w = *reinterpret_cast<const uint4*>(a.g_full + row * kD + 16 * ds + 8 * g);
    }
    qreg[ds] = __builtin_bit_cast(bf16x8, u);
    greg[ds] = __builtin_bit_cast(bf16x8, w);
  }
  const float lse2 = qrow < N ? a.lse2_full[row] : 0.f;
  const float Dq = qrow < N ? a.D_full[row] : 0.f;

  f32x16 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dq[dt] = f32x16{};

  const int j_last = min(N - 1, q0 + kBM - 1) / kBN;

  // HBM -> LDS copy of one K/V tile: each wave moves rows 16*wave .. +15, one
  // 1 KiB instruction per 4 rows; lane l fills physical chunk l % 16 of row
  // 4n + l / 16.  Keys past the end read the last key (masked later).
  auto load_tile = [&](int j, uint16_t* Kd, uint16_t* Vd) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = wave * 4 + r;
      const int rw = 4 * n + (lane >> 4);
      const int p = lane & 15;
      const int64_t key = min(j * kBN + rw, N - 1);
      __builtin_amdgcn_global_load_lds((const glb_void*)(kg + key * kD + 8 * swz_k(rw, p)),
                                       (lds_void*)(Kd + n * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const glb_void*)(vg + key * kD + 8 * swz_k(rw, p)),
                                       (lds_void*)(Vd + n * 512), 16, 0, 0);
    }
  };

  // bucket mask word and entry base of the wave's queries for each half of a
  // tile (uniform): the current tile's, the next one's and the one after
  uint32_t mw[2] = {0u, 0u}, mwn[2] = {0u, 0u}, mwn2[2] = {0u, 0u};
  int mp[2] = {0, 0}, mpn[2] = {0, 0}, mpn2[2] = {0, 0};
  // (vector loads on purpose: a scalar load in flight would turn every wait
  // for an LDS operand into a wait for all of them)
  auto mask_words = [&](int j, uint32_t* m, int* p) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kbase = j * kBN + kh * 32;
      m[kh] = 0u;
      p[kh] = 0;
      if (SPARSE && wave_live && kbase <= wave_last_q) {
        int z = 0;
        asm volatile("" : "+v"(z));
        const int64_t w = ((bc * nb + kbase / block) * G + h % G) * (N / 32) + wave_q0 / 32 + z;
        m[kh] = a.mask[w];
        p[kh] = a.wpos[w];
      }
    }
  };
  // The sparse stream's dS of one half (keys jj*64 + 32 kh ..) for the
  // lanes whose queries selected its block, zero elsewhere.  The rows of the
  // next tile are fetched during the second half of the current one, so they
  // land with the next tile's copies at the barrier: a wait for a register
  // load while tile copies are in flight would wait for those copies too.
  uint4 sd[2][2], sdn[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) sd[kh][0] = sd[kh][1] = sdn[kh][0] = sdn[kh][1] = make_uint4(0, 0, 0, 0);
  auto load_sd = [&](int jj, int kh, uint32_t mword, int mpos, uint4* dst) {
    dst[0] = dst[1] = make_uint4(0, 0, 0, 0);
    const int kbase = jj * kBN + kh * 32;
    const uint32_t m = __builtin_amdgcn_readfirstlane(mword);
    if (wave_live && jj <= j_last && kbase <= wave_last_q && m != 0u && ((m >> col) & 1u)) {
      const int blk = kbase / block;
      // entries of the selected queries below this lane's in the word
      // (lanes 32.. hold the same queries: mbcnt counts the whole word once more)
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u))) -
                        (g ? __builtin_popcount(m) : 0);
      const int e = __builtin_amdgcn_readfirstlane(mpos) + below;
      const uint16_t* src = a.ds_rows + static_cast<int64_t>(e) * block + (kbase - blk * block) + 16 * g;
      dst[0] = *reinterpret_cast<const uint4*>(src);
      dst[1] = *reinterpret_cast<const uint4*>(src + 8);
    }
  };
  auto step = [&](int j, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn) {
    if constexpr (SPARSE) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {       // uniform: scalar registers
        mw[kh] = mwn[kh];
        mp[kh] = mpn[kh];
        mwn[kh] = __builtin_amdgcn_readfirstlane(mwn2[kh]);
        mpn[kh] = __builtin_amdgcn_readfirstlane(mpn2[kh]);
      }
      if (j + 2 <= j_last) mask_words(j + 2, mwn2, mpn2);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        sd[kh][0] = sdn[kh][0];
        sd[kh][1] = sdn[kh][1];
      }
    }
    if (j + 1 <= j_last) load_tile(j + 1, Kn, Vn);
    if (wave_live && j * kBN <= wave_last_q) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int kbase = j * kBN + kh * 32;
        if (kbase > wave_last_q) break;                // uniform: later keys are all masked
        if constexpr (SPARSE) {
          if (kh == 1) {
            load_sd(j + 1, 0, mwn[0], mpn[0], sdn[0]);
            load_sd(j + 1, 1, mwn[1], mpn[1], sdn[1]);
          }
        }
        // ---- S^T = K Q^T, dP^T = V G^T for 32 keys (A: key row kh*32 + col)
        f32x16 s = f32x16{}, dp = f32x16{};
        {
          const int r = kh * 32 + col;
          bf16x8 ok[kD / 16], ov[kD / 16];
          auto rd = [&](int ds) {
            const int off = r * kD + 8 * swz_k(r, 2 * ds + g);
            ok[ds] = lds_read8(&Ks[off]);
            ov[ds] = lds_read8(&Vs[off]);
          };
          rd(0);
#pragma unroll
          for (int ds = 0; ds < kD / 16; ++ds) {      // operands read one step ahead
            __builtin_amdgcn_sched_barrier(0);
            if (ds + 1 < kD / 16) rd(ds + 1);
            s = mfma32x32x16(ok[ds], qreg[ds], s);
            dp = mfma32x32x16(ov[ds], greg[ds], dp);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- dS^T = P^T (dP^T - D); key of register i: kbase + 8(i/4) + 4g + i%4
        const bool diag = kbase + 31 > wave_q0;      // uniform
        // (training modes: plus the sparse stream's dS, element i of its row
        // being the key of register i; it is zero wherever the mask is)
        float dsv[16];
        {
          const uint4 sd0 = sd[kh][0], sd1 = sd[kh][1];
          const uint32_t sw[8] = {sd0.x, sd0.y, sd0.z, sd0.w, sd1.x, sd1.y, sd1.z, sd1.w};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float sp = SPARSE ? __uint_as_float((i & 1) ? (sw[i >> 1] & 0xffff0000u) : (sw[i >> 1] << 16)) : 0.f;
            dsv[i] = fmaf(fast_exp2(s[i] * scale_log2 - lse2), dp[i] - Dq, sp);
          }
        }
        if (diag) {                  // uniform: only the diagonal tiles need the causal mask
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + 4 * g + (i & 3);
            dsv[i] = key <= qrow ? dsv[i] : 0.f;
          }
        }
        // ---- dQ^T += K^T dS^T over the 32 keys (two k-steps of 16)
        bf16x8 bds[2], ka[8];
#pragma unroll
        for (int st = 0; st < 2; ++st)
          bds[st] = to_bf16x8(dsv[8 * st], dsv[8 * st + 1], dsv[8 * st + 2], dsv[8 * st + 3], dsv[8 * st + 4],
                              dsv[8 * st + 5], dsv[8 * st + 6], dsv[8 * st + 7]);
        auto rdk = [&](int u) {
          const int st = u >> 2, dt = u & 3;
          const int r0 = kh * 32 + st * 16 + 4 * gk + srow, r1 = r0 + 8;
          const int c = 4 * dt + 2 * (grp & 1) + (m4 >> 1), e = 4 * (m4 & 1);
          ka[u] = lds_tr_pair(&Ks[r0 * kD + 8 * swz_k(r0, c) + e], &Ks[r1 * kD + 8 * swz_k(r1, c) + e]);
        };
        rdk(0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {                 // K^T read one step ahead
          __builtin_amdgcn_sched_barrier(0);
          if (u + 1 < 8) rdk(u + 1);
          dq[u & 3] = mfma32x32x16(ka[u], bds[u >> 2], dq[u & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);     // the next tile has landed in LDS
    __syncthreads();
  };

  if constexpr (SPARSE) {
    mask_words(0, mwn, mpn);
    if (1 <= j_last) mask_words(1, mwn2, mpn2);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      mwn[kh] = __builtin_amdgcn_readfirstlane(mwn[kh]);
      mpn[kh] = __builtin_amdgcn_readfirstlane(mpn[kh]);
    }
    load_sd(0, 0, mwn[0], mpn[0], sdn[0]);
    load_sd(0, 1, mwn[1], mpn[1], sdn[1]);
  }
  load_tile(0, K0, V0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j <= j_last; j += 2) {
    step(j, K0, V0, K1, V1);
    if (j + 1 > j_last) break;
    step(j + 1, K1, V1, K0, V0);
  }

  // ---- epilogue: dq = scale dQ^T^T, bf16
  if (!wave_live || qrow >= N) return;
  uint16_t* out = static_cast<uint16_t*>(a.dq) + row * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * dt + 8 * i4 + 4 * g;
      *reinterpret_cast<uint2*>(out + d0) =
          make_uint2(pack_bf16x2(scale * dq[dt][4 * i4], scale * dq[dt][4 * i4 + 1]),
                     pack_bf16x2(scale * dq[dt][4 * i4 + 2], scale * dq[dt][4 * i4 + 3]));
    }
}

}  // namespace

void launch_bwd_dq(const Dims& D, const BwdDqArgs& a, hipStream_t s) {
  const int n_qtiles = (D.N + kBM - 1) / kBM;
  dim3 grid(D.B * D.Hq * n_qtiles);   // work items from qtile_item
  timing_begin(kKBwdDq, s);
  if (a.ds_rows)
    hipLaunchKernelGGL(k_bwd_dq<true>, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.nb, D.block, D.scale,
                       D.scale * 1.4426950408889634f, n_qtiles);
  else
    hipLaunchKernelGGL(k_bwd_dq<false>, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.nb, D.block, D.scale,
                       D.scale * 1.4426950408889634f, n_qtiles);
  timing_end(kKBwdDq, s);
}

}  // namespace ssa
