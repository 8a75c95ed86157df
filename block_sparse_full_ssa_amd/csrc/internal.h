// Internal launch interface between the C entry points (api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssa {

// Validated layer dimensions.
struct Dims {
  int B, Hq, Hkv, G, N, d, block, nb, K;
  int dtype;        // 0 fp32, 1 bf16
  float scale;      // softmax scale on q.k
  // Query rows per head and the position of row 0.  A layer has Nq = N and
  // q_off = 0; a prefill chunk has Nq rows at positions q_off .. q_off+Nq-1
  // against N = the cache's capacity (keys at positions 0 .. q_off+Nq-1).
  int Nq = 0, q_off = 0;
  int64_t rows() const { return static_cast<int64_t>(B) * Hq * Nq; }
  int64_t q_elems() const { return rows() * d; }
  int64_t kv_elems() const { return static_cast<int64_t>(B) * Hkv * N * d; }
};

enum Mode { kDualFull = 0, kDualSparse = 1, kFullOnly = 2, kSparseOnly = 3 };

// Kernel identifiers for the optional event timing.
enum KernelId {
  kKBlockMean = 0,
  kKSelect,
  kKFwdSimt,
  kKFwdMfma,
  kKLossReduce,
  kKBwdPre,
  kKBwdSimt,
  kKBwdMfma,
  kKConvert,
  kKZero,
  kKBucket,
  kKSparsePart,
  kKSparseMerge,
  kKBwdSparse,
  kKBwdDq,
  kKProbeMfma,
  kKProbeCopy,
  kKDecode,
  kKDqMerge,
  kKProbeAtomic,
  kKProbeLds,
  kKernelCount
};

// Timing hooks (api.hip); no-ops unless timing is enabled.
void timing_begin(int kernel, hipStream_t s);
void timing_end(int kernel, hipStream_t s);
// While a TimingPause lives, the calling thread records no events (entry
// points that must not create HIP objects).
struct TimingPause {
  TimingPause();
  ~TimingPause();
};
// Sets the text that ssa_last_error() reports on this thread.
void set_last_error(const char* msg);

// --- selection (select.hip) ---
void launch_block_mean(const Dims& D, const void* k, float* mu, hipStream_t s);
// split: select_split_bytes(D) of workspace (bf16 layers: the two-term bf16
// split of the means that the matrix scoring reads).
size_t select_split_bytes(const Dims& D);
void launch_select(const Dims& D, const void* q, const float* mu, uint16_t* split, int32_t* sel, hipStream_t s);

// --- generic SIMT kernels (simt.hip): every supported shape, fp32 and bf16 ---
struct FwdArgs {
  const void *q, *k, *v;
  const int32_t* sel;
  void *h_full, *h_sparse;
  float *lse_full, *lse_sparse, *delta;
  float* row_sq;     // per-row sum of (h_full - h_sparse)^2, dual modes only
  int mode;
  // optional full-stream diagnostics per row [B, Hq, N]: probability mass on
  // the first key block, entropy (nats); both null or both set
  float* sink_mass = nullptr;
  float* entropy = nullptr;
};
void launch_fwd_simt(const Dims& D, const FwdArgs& a, hipStream_t s);

struct BwdArgs {
  const void *q, *k, *v;
  const int32_t* sel;
  const void *h_full, *h_sparse;
  const float *lse_full, *lse_sparse;
  const void* dout;
  void* dq;           // SIMT: written directly in dtype
  float *dk_acc, *dv_acc;  // fp32 accumulators [B,Hkv,N,d], zeroed first
  float w_sparsity, w_commit;
  int mode;
};
void launch_bwd_simt(const Dims& D, const BwdArgs& a, hipStream_t s);

// --- bf16 MFMA kernels ---
bool fwd_mfma_supported(const Dims& D);
// dual and FULL_ONLY modes; returns the status of the LDS grant (the launch's
// own status comes from hipGetLastError)
hipError_t launch_fwd_mfma(const Dims& D, const FwdArgs& a, hipStream_t s);

struct BwdPreArgs {
  const void* dout;                 // may be null: zero upstream gradient
  const void *h_full, *h_sparse;
  const float *lse_full, *lse_sparse;
  uint16_t *g_full, *g_sparse;      // bf16 stream gradients [rows][d]
  float *D_full, *D_sparse;         // rowsum(G o h)
  float *lse2_full, *lse2_sparse;   // lse * log2(e)
  // per row of the full stream, the dK / dV kernel's row operands: -lse2 / c
  // (c = scale * log2(e)) and -D, each split into three bf16 terms t0, t1, t2
  // with t0 + t1 + t2 equal to the value up to 2^-24 of it, stored as
  // {t0 | t1 << 16, t2} per value
  uint4* rowv_full;
  int mode;
};
// Full-stream backward: G_f, D_f, lse2_f of every row.
struct BwdMainArgs {                // dK, dV
  const void *q, *k, *v;
  const uint16_t* g_full;
  const uint4* rowv_full;           // BwdPreArgs::rowv_full
  void *dk, *dv;
  const float *dk_part, *dv_part;   // fp32 sparse-stream dK / dV to add (training modes) or null
};
struct BwdDqArgs {                  // dQ
  const void *q, *k, *v;
  const uint16_t* g_full;
  const float *lse2_full, *D_full;
  // training modes: the sparse stream's buckets and dS rows (bf16 [bucket
  // entries][block], 32-key groups in the kernel's lane order), added to the
  // full stream's dS before the dQ product; null for the full stream alone
  const uint32_t* mask;
  const int32_t* wpos;
  const uint16_t* ds_rows;
  void* dq;
};
void launch_bwd_dq(const Dims& D, const BwdDqArgs& a, hipStream_t s);
bool bwd_mfma_supported(const Dims& D);
void launch_bwd_pre(const Dims& D, const BwdPreArgs& a, float w_sparsity, float w_commit, hipStream_t s);
void launch_bwd_mfma(const Dims& D, const BwdMainArgs& a, hipStream_t s);

// --- key-block buckets (bucket.hip) ---
struct Buckets {
  uint32_t* mask;    // [B*Hkv][nb][G][N/32] row masks of each bucket
  int32_t* count;    // [B*Hkv*nb] rows per bucket
  int32_t* offs;     // [B*Hkv*nb + 1] exclusive prefix of count
  int32_t* rows;     // entries (h % G) * N + t, bucket after bucket
  int32_t* wpos;     // [as mask] position in rows of each mask word's first entry
};
int64_t bucket_mask_words(const Dims& D);
int64_t bucket_capacity(const Dims& D);   // upper bound on the entries: rows * min(K, nb)
void launch_buckets(const Dims& D, const int32_t* sel, const Buckets& bk, hipStream_t s);

// --- sparse-only forward on buckets (sparse_fwd.hip) ---
struct SparseFwdArgs {
  const void *q, *k, *v;
  const int32_t* sel;
  const uint32_t* mask;                 // buckets
  const int32_t *offs, *rows, *wpos;
  uint16_t* part_o;                     // [bucket capacity + 1][d] bf16 partial outputs, bucket order
  float* part_lse;                      // [bucket capacity + 1] partial log-sum-exps (log2 units)
  void* h_sparse;
  float* lse_sparse;                    // may be null
};
bool sparse_fwd_supported(const Dims& D);
void launch_sparse_fwd(const Dims& D, const SparseFwdArgs& a, hipStream_t s);

// --- sparse-stream backward on buckets (sparse_bwd.hip) ---
struct SparseBwdArgs {
  const void *q, *k, *v;
  const int32_t *offs, *rows;           // buckets
  const uint16_t* g_sparse;             // bf16 G_s [rows][d]
  const float *lse2_sparse, *D_sparse;
  uint16_t* dq_part;                    // sparse-only: bf16 [bucket entries][d] partial dQ rows
  uint16_t* ds_rows;                    // bf16 [bucket entries][block] dS rows for the dQ kernel, or null
  float *dk_part, *dv_part;             // fp32 [B*Hkv][N][d] results, or null: write dk, dv (bf16)
  void *dk, *dv;
};
bool sparse_bwd_supported(const Dims& D);
void launch_bwd_sparse(const Dims& D, const SparseBwdArgs& a, hipStream_t s);
// sparse-only dQ: each row's partials summed over its selected blocks -> dq (bf16)
void launch_sparse_dq_merge(const Dims& D, const int32_t* sel, const uint32_t* mask, const int32_t* wpos,
                            const uint16_t* part, void* dq, hipStream_t s);

// --- small kernels (misc.hip) ---
void launch_zero_f32(float* p, int64_t n, hipStream_t s);
void launch_convert(const float* src, void* dst, int dtype, int64_t n, hipStream_t s);
size_t loss_scratch_bytes();
// Machine probes (measurement only): a dense bf16 matrix-core loop of
// blocks x 4 waves x 4 chains x iters products, and a device copy of `bytes`
// (a multiple of 16).
// Single-token decode over a KV cache (D.N = cache capacity, D.nb its blocks).
constexpr int kDecodeChunk = 16;         // blocks per part of the full stream
struct DecodeArgs {
  const void* q;             // [B, Hq, d]
  const void *k, *v;         // caches [B, Hkv, N, d]
  const float* mu;           // block-mean cache [B, Hkv, nb, d] (sparse)
  const int32_t* pos;        // [B] position of the new token (keys 0..pos)
  int32_t* sel;              // [B, Hq, K] selection (sparse), null for the full stream
  uint32_t* codes;           // workspace (sparse): score codes [B*Hq][nb]
  float *part_o, *part_ml;   // workspace: parts' outputs [B*Hq][P][d], (max, sum) [B*Hq][P][2]
  void* h;                   // [B, Hq, d]
  float* lse;                // [B, Hq] or null
};
int decode_parts(const Dims& D, bool sparse);
void launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t s);
void launch_cache_means(const Dims& D, const void* k, float* mu, int j0, int j1, hipStream_t s);

// Per-head means over the N rows of two per-row arrays [B*Hq][N] -> out [B*Hq][2].
void launch_head_means(const float* a, const float* b, int64_t n_heads, int N, float* out, hipStream_t s);
void launch_probe_mfma(float* sink, int blocks, int iters, hipStream_t s);
void launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
void launch_probe_atomic(float* buf, int ntiles, int blocks, int iters, hipStream_t s);
void launch_probe_lds(float* sink, int blocks, int iters, int mode, hipStream_t s);
void launch_loss_reduce(const float* row_sq, int64_t n_rows, double inv_count, double* scratch, float* losses,
                        hipStream_t s);

}  // namespace ssa
