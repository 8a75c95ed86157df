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
// query's row is entry wpos + popcount of the word's lower bits.  With 64-key
// blocks (one block per tile) the selected queries' rows of a tile are
// consecutive entries, so a wave copies them HBM -> LDS with the next tile
// (up to 12 rows; a wave with more reads the rest from HBM when it uses
// them); other block sizes load each selected lane's part of its row into
// registers during the previous tile.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace ssa {
namespace {

constexpr int kBM = 128;         // queries per workgroup
constexpr int kBN = 64;          // keys per tile


// Physical 16-byte chunk of logical chunk c in a K / V row r of 2 HD bytes (K
// is read by rows and by transposes): swz256 for 256-byte rows (HD = 128),
// swz128 for 128-byte rows (HD = 64).
template <int HD> __device__ __forceinline__ int swz_k(int r, int c) {
  return HD == 128 ? swz256(r, c) : swz128(r, c);
}

// SP: 0 the full stream alone; 1 with the sparse stream's dS rows through
// registers (any block size); 2 through LDS (64-key blocks).  HD: head dimension.
template <int SP, int HD>
__global__ void __launch_bounds__(256, 2)
    k_bwd_dq(BwdDqArgs a, int Hq, int G, int N, int nb, int block, float scale, float scale_log2, int n_qtiles,
             int64_t ds_elems) {
  constexpr bool SPARSE = SP != 0;
  constexpr int kD = HD;
  constexpr int kDT = HD / 32;                 // 32-column tiles of dQ
  constexpr int kTile = kBN * kD;
  __shared__ __attribute__((aligned(16))) uint16_t K0[kTile], K1[kTile], V0[kTile], V1[kTile];
  // SP = 2: each wave's first kSDRows dS rows of the current / next tile
  constexpr int kSDRows = 12;
  constexpr int kSD = SP == 2 ? 4 * kSDRows * kBN : 8;
  __shared__ __attribute__((aligned(16))) uint16_t SD0[kSD], SD1[kSD];
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
  // dP^T starts at -D of the lane's query: one extra product, -D as three
  // bf16 terms in the k-slots 0..2 of the B operand (lanes of k-group 0)
  // against ones in the same k-slots of the A operand, so that dS needs no
  // per-element subtraction
  bf16x8 dterm, ones;
  {
    const uint2 t = split3_bf16(-(qrow < N ? a.D_full[row] : 0.f));
    dterm = __builtin_bit_cast(bf16x8, g ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(t.x, t.y, 0u, 0u));
    ones = __builtin_bit_cast(bf16x8, g ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(0x3F803F80u, 0x00003F80u, 0u, 0u));
  }

  f32x16 dq[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) dq[dt] = f32x16{};

  const int j_last = min(N - 1, q0 + kBM - 1) / kBN;

  // HBM -> LDS copy of one K/V tile: each wave moves a quarter of its rows,
  // one 1 KiB instruction per kRowsOp rows; lane l fills physical chunk
  // l % (HD / 8) of row kRowsOp n + l / (HD / 8) (byte offsets within the
  // tile, fixed per lane).  Keys past the end lie outside the tile's buffer
  // resource and read zeros (masked later).
  constexpr int kRowsOp = 512 / HD;
  constexpr int kOps = kBN / kRowsOp / 4;
  uint32_t toff[kOps];
#pragma unroll
  for (int r = 0; r < kOps; ++r) {
    const int rw = kRowsOp * (wave * kOps + r) + lane / (HD / 8);
    toff[r] = 2 * (rw * kD + 8 * swz_k<HD>(rw, lane % (HD / 8)));
  }
  auto load_tile = [&](int j, uint16_t* Kd, uint16_t* Vd) {
    const int k0 = j * kBN;
    const uint32_t bytes = static_cast<uint32_t>(min(kBN, N - k0)) * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg + static_cast<int64_t>(k0) * kD, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vg + static_cast<int64_t>(k0) * kD, bytes);
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      const int n = wave * kOps + r;
      buffer_to_lds16(rk, Kd + n * 512, toff[r]);
      buffer_to_lds16(rv, Vd + n * 512, toff[r]);
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
  // (SP = 1 only: the arrays are unused otherwise)
  constexpr int kSdH = SP == 1 ? 2 : 1;
  uint4 sd[kSdH][2], sdn[kSdH][2];
#pragma unroll
  for (int kh = 0; kh < kSdH; ++kh) sd[kh][0] = sd[kh][1] = sdn[kh][0] = sdn[kh][1] = make_uint4(0, 0, 0, 0);
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
  // SP = 2: the dS rows of the wave's selected queries of a tile (its mask
  // word and entry position, uniform) -> LDS, at most kSDRows of them; the
  // resource ends with the buffer, so parts past it read zeros (rows past
  // the tile's are never read)
  auto copy_rows = [&](uint32_t word, int pos, uint16_t* SDd) {
    uint16_t* dst = SDd + wave * kSDRows * kBN;
    const int cnt = __builtin_popcount(word);
    const int64_t base = static_cast<int64_t>(pos) * kBN;
    const int64_t left = ds_elems - base;          // elements from the first row to the buffer's end
    const int64_t span = left < kSDRows * kBN ? (left > 0 ? left : 0) : kSDRows * kBN;
    const __amdgpu_buffer_rsrc_t rr = tile_rsrc(a.ds_rows + base, static_cast<uint32_t>(span) * 2);
#pragma unroll
    for (int u = 0; u < (kSDRows * kBN * 2 + 1023) / 1024; ++u) {
      if (u * 8 < cnt && u * 1024 + 16 * lane < kSDRows * kBN * 2)
        buffer_to_lds16(rr, dst + u * 512, static_cast<uint32_t>(u * 1024 + 16 * lane));
    }
  };
  // HD = 128: byte offsets of the K / V row reads of d-steps 0..3 (key row
  // col; rows 32 further share the swizzle, and d-step ds + 4 flips bit 7:
  // its logical chunk 2 ds + g flips bit 3, and so does the physical one) and
  // of the K^T transpose reads of rows 4 gk + srow and 8 further (column tile
  // dt: an XOR of 64 dt, the swizzle's 32 srow kept apart on bits 5 and 6,
  // which the rest leaves clear), held in registers
  constexpr int kRO = kD / 32, kFlip = kD;   // (HD = 128: 4 offsets, bit 7; HD = 64: 2, bit 6)
  int roff[kRO], tk[2];
#pragma unroll
  for (int ds = 0; ds < kRO; ++ds) roff[ds] = 2 * (col * kD + 8 * swz_k<HD>(col, 2 * ds + g));
  {
    // (HD = 64: swizzle term 4 ((srow / 2) % 2) + gk (+ 2))
    const int y = 2 * (grp & 1) + (m4 >> 1), e4 = 4 * (m4 & 1);
    const int t = HD == 128 ? srow : (srow >> 1) & 1;
    tk[0] = 2 * ((4 * gk + srow) * kD + 8 * (y ^ gk) + e4 + 32 * t);
    tk[1] = 2 * ((4 * gk + srow + 8) * kD + 8 * (y ^ (gk + 2)) + e4 + 32 * t);
  }
  auto rd16 = [](const uint16_t* base, int off) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off));
  };
  auto step = [&](int j, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn, const uint16_t* SDs,
                  uint16_t* SDn) {
    if constexpr (SPARSE) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {       // uniform: scalar registers
        mw[kh] = mwn[kh];
        mp[kh] = mpn[kh];
        mwn[kh] = __builtin_amdgcn_readfirstlane(mwn2[kh]);
        mpn[kh] = __builtin_amdgcn_readfirstlane(mpn2[kh]);
      }
      if (j + 2 <= j_last) mask_words(j + 2, mwn2, mpn2);
    }
    if constexpr (SP == 1) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        sd[kh][0] = sdn[kh][0];
        sd[kh][1] = sdn[kh][1];
      }
    }
    if (j + 1 <= j_last) load_tile(j + 1, Kn, Vn);
    if constexpr (SP == 2) {
      if (wave_live && j + 1 <= j_last && mwn[0] != 0u) copy_rows(mwn[0], mpn[0], SDn);
    }
    if (wave_live && j * kBN <= wave_last_q) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int kbase = j * kBN + kh * 32;
        if (kbase > wave_last_q) break;                // uniform: later keys are all masked
        if constexpr (SP == 1) {
          if (kh == 1) {
            load_sd(j + 1, 0, mwn[0], mpn[0], sdn[0]);
            load_sd(j + 1, 1, mwn[1], mpn[1], sdn[1]);
          }
        }
        // ---- S^T = K Q^T, dP^T = V G^T for 32 keys (A: key row kh*32 + col)
        f32x16 s = f32x16{}, dp = mfma32x32x16(ones, dterm, f32x16{});
        {
          const int r = kh * 32 + col;
          bf16x8 ok[kD / 16], ov[kD / 16];
          auto rd = [&](int ds) {
            const int o = (ds < kRO ? roff[ds] : roff[ds - kRO] ^ kFlip) + 2 * kD * kh * 32;
            ok[ds] = rd16(Ks, o);
            ov[ds] = rd16(Vs, o);
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
        // K^T operands of the dQ products (step u: k-step u / kDT, column
        // tile u % kDT); the first two are read during dS
        bf16x8 ka[2 * kDT];
        auto rdk = [&](int u) {
          const int st = u / kDT, dt = u % kDT;
          const int rb = 2 * kD * (kh * 32 + st * 16);
          const char* kb = reinterpret_cast<const char*>(Ks);
          ka[u] = lds_tr_pair(reinterpret_cast<const uint16_t*>(kb + ((tk[0] ^ (64 * dt)) + rb)),
                              reinterpret_cast<const uint16_t*>(kb + ((tk[1] ^ (64 * dt)) + rb)));
        };
        rdk(0);
        rdk(1);
        __builtin_amdgcn_sched_barrier(0);
        // ---- dS^T = P^T (dP^T - D); key of register i: kbase + 8(i/4) + 4g + i%4
        const bool diag = kbase + 31 > wave_q0;      // uniform
        // (training modes: plus the sparse stream's dS, element i of its row
        // being the key of register i; it is zero wherever the mask is)
        float dsv[16];
        {
          uint4 sd0 = make_uint4(0, 0, 0, 0), sd1 = make_uint4(0, 0, 0, 0);
          if constexpr (SP == 1) {
            sd0 = sd[kh][0];
            sd1 = sd[kh][1];
          } else if constexpr (SP == 2) {
            const uint32_t m = mw[0];        // (one block per tile: both halves' word)
            if (m != 0u) {                   // uniform
              const bool mine = (m >> col) & 1u;
              const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u))) -
                                (g ? __builtin_popcount(m) : 0);
              if (mine && below < kSDRows) {
                const uint16_t* src = SDs + (wave * kSDRows + below) * kBN + kh * 32 + 16 * g;
                sd0 = *reinterpret_cast<const uint4*>(src);
                sd1 = *reinterpret_cast<const uint4*>(src + 8);
              }
              if (__builtin_popcount(m) > kSDRows) {   // uniform, rare: the rest from HBM
                if (mine && below >= kSDRows) {
                  const uint16_t* src = a.ds_rows + static_cast<int64_t>(mp[0] + below) * kBN + kh * 32 + 16 * g;
                  sd0 = *reinterpret_cast<const uint4*>(src);
                  sd1 = *reinterpret_cast<const uint4*>(src + 8);
                }
                // (waited for here, so that no other tile's use of the rows waits)
                __builtin_amdgcn_s_waitcnt(0);
              }
            }
          }
          const uint32_t sw[8] = {sd0.x, sd0.y, sd0.z, sd0.w, sd1.x, sd1.y, sd1.z, sd1.w};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float sp = SPARSE ? __uint_as_float((i & 1) ? (sw[i >> 1] & 0xffff0000u) : (sw[i >> 1] << 16)) : 0.f;
            dsv[i] = fmaf(fast_exp2(s[i] * scale_log2 - lse2), dp[i], sp);
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
        bf16x8 bds[2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
          bds[st] = to_bf16x8(dsv[8 * st], dsv[8 * st + 1], dsv[8 * st + 2], dsv[8 * st + 3], dsv[8 * st + 4],
                              dsv[8 * st + 5], dsv[8 * st + 6], dsv[8 * st + 7]);
#pragma unroll
        for (int u = 0; u < 2 * kDT; ++u) {           // K^T read two steps ahead
          __builtin_amdgcn_sched_barrier(0);
          if (u + 2 < 2 * kDT) {
            rdk(u + 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // the reads, then the product
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          dq[u % kDT] = mfma32x32x16(ka[u], bds[u / kDT], dq[u % kDT]);
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
    if constexpr (SP == 1) {
      load_sd(0, 0, mwn[0], mpn[0], sdn[0]);
      load_sd(0, 1, mwn[1], mpn[1], sdn[1]);
    } else {
      if (wave_live && mwn[0] != 0u) copy_rows(mwn[0], mpn[0], SD0);
    }
  }
  load_tile(0, K0, V0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j <= j_last; j += 2) {
    step(j, K0, V0, K1, V1, SD0, SD1);
    if (j + 1 > j_last) break;
    step(j + 1, K1, V1, K0, V0, SD1, SD0);
  }

  // ---- epilogue: dq = scale dQ^T^T, bf16
  if (!wave_live || qrow >= N) return;
  uint16_t* out = static_cast<uint16_t*>(a.dq) + row * kD;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
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
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a, D.Hq, D.G, D.N, D.nb, D.block, D.scale,
                       D.scale * 1.4426950408889634f, n_qtiles, a.ds_rows ? bucket_capacity(D) * D.block : int64_t{0});
  };
  auto by_mode = [&](auto hd_tag) {
    constexpr int HD = decltype(hd_tag)::value;
    if (!a.ds_rows) go(k_bwd_dq<0, HD>);
    else if (D.block == kBN) go(k_bwd_dq<2, HD>);
    else go(k_bwd_dq<1, HD>);
  };
  if (D.d == 64) by_mode(std::integral_constant<int, 64>{});
  else by_mode(std::integral_constant<int, 128>{});
  timing_end(kKBwdDq, s);
}

}  // namespace ssa
