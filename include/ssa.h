/*
 * ssa.h -- C interface of libssa: SSA (Sparse Sparse Attention) dual-stream
 * causal attention for AMD Instinct MI355X (gfx950).
 *
 * SSA trains one attention layer in two streams over the same q, k, v
 * (arXiv 2511.20102, "SSA: Sparse Sparse Attention by Aligning Full and Sparse
 * Attention Outputs in Feature Space"; Sintesi Tecnica, section 2):
 *   - the full stream: causal softmax attention over every earlier key;
 *   - the sparse stream: block-sparse attention, each query restricted to the
 *     keys of its selected key blocks and renormalised over them;
 *   - per training step one stream is drawn as the active one; the other
 *     (counterpart) output serves only the alignment losses and receives no
 *     upstream gradient;
 *   - L_sparsity pulls h_full toward a fixed h_sparse, L_commit pulls h_sparse
 *     toward a fixed h_full; their sum is L_align in the total objective.
 * The discarded mass delta(t) is the full-attention probability of query t
 * that falls on keys outside its sparse support (Sintesi Tecnica, section 2,
 * 'Allineamento Bidirezionale'; the error of sparse attention grows linearly
 * with it, section 1).
 *
 * Block selection (the pages leave it open; fixed here): for query t in block
 * i_t = t / block, every earlier block j < i_t scores q_t . mean(k over block
 * j) in fp32; the own block i_t is always kept; the top_k - 1 best-scoring
 * earlier blocks complete the set, the lower index winning a tie.
 *
 * Conventions shared by every entry point
 *   Layout     q, h_full, h_sparse, d_out, dq: [B, Hq, N, d] contiguous;
 *              k, v, dk, dv: [B, Hkv, N, d] with Hkv = Hq / group;
 *              query head h reads KV head h / group.
 *              lse_full, lse_sparse, delta: [B, Hq, N] fp32.
 *              sel: [B, Hq, N, top_k] int32, each row ascending block indices
 *              followed by -1 padding (a row of block i holds min(top_k, i+1)
 *              entries).
 *   dtype      SSA_BF16: q/k/v/outputs/gradients bf16 (bf16 MFMA, fp32
 *              accumulation); SSA_F32: all fp32 (fp32 arithmetic throughout).
 *   Logits     z = softmax_scale * q . k, causal (key index <= query index);
 *              softmax_scale <= 0 selects 1/sqrt(d).  lse = log sum exp z over
 *              the stream's keys (natural log).
 *   Pointers   All tensor pointers are DEVICE pointers owned by the caller.
 *              The library allocates no device memory: every scratch buffer
 *              lives in the caller's workspace ``ws`` of ``ws_bytes`` bytes,
 *              sized by ssa_workspace_size() and aligned to 256 bytes.
 *   Streams    ``stream`` is a hipStream_t (NULL = the null stream).  Every
 *              call only enqueues work on it and returns; results are valid
 *              once the stream has reached that point.
 *   Errors     Arguments are validated on the host before anything is
 *              enqueued; an invalid call returns a status other than SSA_OK
 *              and enqueues nothing.  SSA_ERR_HIP reports a failed launch
 *              (details in ssa_last_error()).  No C++ exception crosses this
 *              interface.  Calls on different streams may run concurrently if
 *              their workspaces differ.
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_ERR_NULL = 1,        /* a required pointer is NULL */
  SSA_ERR_SHAPE = 2,       /* inconsistent sizes (group, N % block, top_k < 1, ...) */
  SSA_ERR_UNSUPPORTED = 3, /* valid but not implemented (head_dim, block, dtype) */
  SSA_ERR_WORKSPACE = 4,   /* ws_bytes below ssa_workspace_size() or ws misaligned */
  SSA_ERR_HIP = 5          /* the HIP runtime reported an error */
} ssa_status_t;

typedef enum { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype_t;

/* Which outputs exist and where the upstream gradient goes. */
typedef enum {
  SSA_DUAL_ACTIVE_FULL = 0,   /* training step, full stream active   */
  SSA_DUAL_ACTIVE_SPARSE = 1, /* training step, sparse stream active */
  SSA_FULL_ONLY = 2,          /* full attention alone                */
  SSA_SPARSE_ONLY = 3         /* block-sparse attention alone        */
} ssa_mode_t;

typedef enum { SSA_OP_SELECT = 0, SSA_OP_FWD = 1, SSA_OP_BWD = 2, SSA_OP_DECODE = 3 } ssa_op_t;

typedef struct {
  int32_t batch;          /* B >= 1                                  */
  int32_t heads_q;        /* Hq >= 1                                 */
  int32_t group;          /* G = Hq / Hkv >= 1, divides Hq           */
  int32_t seqlen;         /* N >= block, N % block == 0,
                             N / block <= 4096 (else UNSUPPORTED)   */
  int32_t head_dim;       /* d: 64 or 128                            */
  int32_t block;          /* key block size: 32, 64 or 128           */
  int32_t top_k;          /* selected blocks per query incl. own, >= 1;
                             larger than N/block selects every block */
  float softmax_scale;    /* <= 0: 1/sqrt(d)                         */
  int32_t dtype;          /* ssa_dtype_t                             */
} ssa_shape_t;

/* Bytes of workspace that ``op`` needs for ``shape`` in ``mode`` (0 on an
 * invalid shape, or when the op needs none).  SSA_OP_SELECT / _FWD / _BWD
 * size the layer entry points; SSA_OP_DECODE sizes ssa_decode for a cache
 * of capacity shape->seqlen (modes SSA_FULL_ONLY and SSA_SPARSE_ONLY only).
 * A prefill chunk is sized by ssa_prefill_workspace_size.  A workspace of
 * this size may be reused across calls that are ordered on one stream. */
size_t ssa_workspace_size(const ssa_shape_t* shape, int32_t mode, int32_t op);

/*
 * Block selection (the rule in the header comment).
 *   q [B,Hq,N,d], k [B,Hkv,N,d] in shape->dtype  -> sel [B,Hq,N,top_k] int32.
 * Block means are accumulated in fp32.  Scores of fp32 layers are fp32 dot
 * products; those of bf16 layers multiply q (exact) by each mean split into
 * two bf16 terms (hi = bf16(mu), lo = bf16(mu - hi), together within 2^-18
 * of mu relative) with exact products and fp32 sums.  A cutoff whose two
 * scores differ by less than this rounding may rank either way.
 * Workspace: the fp32 block means and, for bf16, their two-term split.
 */
ssa_status_t ssa_select_blocks(const ssa_shape_t* shape, const void* q, const void* k,
                               int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward of one SSA layer (Sintesi Tecnica, section 2).
 *   Dual modes: writes h_full, h_sparse (dtype), lse_full, lse_sparse,
 *     delta (fp32 [B,Hq,N]; delta = 1 - exp(lse_sparse - lse_full)) and
 *     losses[2] = {L_sparsity, L_commit} (fp32, device), each the mean of
 *     (h_full - h_sparse)^2 over all B*Hq*N*d elements, accumulated from the
 *     fp32 outputs before rounding.  The two values are equal; they differ
 *     only in their gradients.  sel is required.
 *   SSA_FULL_ONLY: writes h_full, lse_full; sel, h_sparse, lse_sparse, delta
 *     and losses may be NULL and are not touched.
 *   SSA_SPARSE_ONLY: writes h_sparse, lse_sparse; h_full, lse_full, delta and
 *     losses may be NULL.  Computed key-block-stationary: the rows that
 *     selected each key block are gathered, each (row, selected block) gets a
 *     partial result and the partials are merged by their log-sum-exps, so
 *     the work follows the selected pairs.
 * In every mode the non-negative entries of a row of sel must be ascending,
 *   as ssa_select_blocks writes them.  Entries that name no causal block of
 *   the row (negative, above the row's own block, or >= N / block) are
 *   ignored wherever they stand, and so is an entry equal to the one before
 *   it.
 * lse pointers may be NULL when the caller will not run the backward.
 */
ssa_status_t ssa_attn_fwd(const ssa_shape_t* shape, int32_t mode, const void* q,
                          const void* k, const void* v, const int32_t* sel, void* h_full,
                          void* h_sparse, float* lse_full, float* lse_sparse, float* delta,
                          float* losses, void* ws, size_t ws_bytes, void* stream);

/*
 * ssa_attn_fwd plus diagnostics of the full-attention distribution p_full,
 * computed in the same pass.  The pages track how much attention lands on
 * the sink area at the start of the sequence (English abstract, last
 * sentence) and how sparse the attention is (Sintesi Tecnica, section 5,
 * 'Sparsita Intrinseca') without defining a statistic; the ones written here:
 *   sink_mass [B,Hq,N] fp32: sum of p_full(t, i) over the first key block
 *     (keys i < block);
 *   entropy   [B,Hq,N] fp32: -sum_i p_full(t, i) ln p_full(t, i) (nats) over
 *     the causal keys;
 *   head_stats [B,Hq,2] fp32 (optional, NULL to skip): the mean over the N
 *     rows of sink_mass and of entropy, per head.
 * Modes with the full stream only (dual, SSA_FULL_ONLY): SSA_SPARSE_ONLY
 * returns SSA_ERR_UNSUPPORTED.  sink_mass and entropy are required
 * (SSA_ERR_NULL).  All other arguments, the workspace size and the errors are
 * those of ssa_attn_fwd.
 */
ssa_status_t ssa_attn_fwd_stats(const ssa_shape_t* shape, int32_t mode, const void* q,
                                const void* k, const void* v, const int32_t* sel, void* h_full,
                                void* h_sparse, float* lse_full, float* lse_sparse, float* delta,
                                float* losses, float* sink_mass, float* entropy, float* head_stats,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of one SSA layer.  With M = B*Hq*N*d the gradients reaching the
 * two outputs are
 *   G_full   = [active = full]   d_out + w_sparsity (2/M) (h_full - h_sparse)
 *   G_sparse = [active = sparse] d_out + w_commit   (2/M) (h_sparse - h_full)
 * in the dual modes (stop-gradient targets: Sintesi Tecnica section 2, items
 * 1 and 2 of 'Allineamento Bidirezionale'); single-stream modes take
 * G = d_out for their one stream and ignore the weights.  Then for each
 * stream with probabilities p (recomputed from q, k and the stored lse):
 *   dq_t = scale sum_i p_ti (G_t.v_i - G_t.h_t) k_i,  dk_i = scale sum_t (same) q_t,
 *   dv_i = sum_t p_ti G_t, summed over both streams and, for dk/dv, over the
 *   query heads of a group.  No gradient flows through the selection.
 * Inputs are the forward's q, k, v, sel and outputs (h_* and lse_* of the
 * streams the mode has; the others may be NULL).  d_out may be NULL for a
 * zero upstream gradient.  Writes dq [B,Hq,N,d], dk, dv [B,Hkv,N,d] (dtype),
 * overwriting them.
 */
ssa_status_t ssa_attn_bwd(const ssa_shape_t* shape, int32_t mode, float w_sparsity,
                          float w_commit, const void* q, const void* k, const void* v,
                          const int32_t* sel, const void* h_full, const void* h_sparse,
                          const float* lse_full, const float* lse_sparse, const void* d_out,
                          void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * ssa_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, hosts that forbid allocation).  Arguments, outputs and errors are
 * those of ssa_attn_fwd; the same kernels run.  Their workspace comes from a
 * static device array of ssa_noalloc_scratch_bytes() bytes (16 MiB), one per
 * device, held until the process ends: a layer whose
 * ssa_workspace_size(shape, mode, SSA_OP_FWD) exceeds it returns
 * SSA_ERR_WORKSPACE and enqueues nothing.  (Dual modes need 4 bytes per query
 * row, so up to about four million rows B*Hq*N; SSA_FULL_ONLY needs none;
 * SSA_SPARSE_ONLY fits only small layers.)  Nothing is allocated and no HIP
 * event is created, also with timing enabled; the first call on a device
 * looks up the array's device address.  Every call on one device shares the
 * array: calls that may overlap in time on one device (different streams or
 * threads) race and must be ordered by the caller.
 */
size_t ssa_noalloc_scratch_bytes(void);
ssa_status_t ssa_attn_fwd_noalloc(const ssa_shape_t* shape, int32_t mode, const void* q,
                                  const void* k, const void* v, const int32_t* sel, void* h_full,
                                  void* h_sparse, float* lse_full, float* lse_sparse, float* delta,
                                  float* losses, void* stream);

/* Static text for a status code. */
const char* ssa_status_string(int32_t status);

/* Details of the last error returned on this thread ("" if none). */
const char* ssa_last_error(void);

/*
 * Kernel timing for measurement harnesses.  While enabled, the library
 * records a HIP event pair on the launch stream around every launch of its
 * kernels.  ssa_timing_query() waits for the recorded events and returns the
 * summed duration (ms) and launch count of one kernel, by name as returned
 * by ssa_kernel_name(i) for i = 0 .. ssa_kernel_count()-1.  Enabling clears
 * earlier records.  Off by default.  These records are the library's only
 * process-wide host state (guarded by a mutex; while enabled, launches from
 * several threads all record into them); with timing off every entry point is
 * reentrant.  Each record creates two HIP events, so harnesses should time
 * headline wall-clock figures with timing off.
 */
ssa_status_t ssa_timing_enable(int32_t enabled);
ssa_status_t ssa_timing_query(const char* kernel, double* total_ms, int64_t* launches);
int32_t ssa_kernel_count(void);
const char* ssa_kernel_name(int32_t i);

/*
 * Inference over a KV cache (Sintesi Tecnica, section 4, 'Efficienza': at
 * inference SSA performs MoBA's operations, i.e. the sparse stream alone).
 * The shape describes the cache: seqlen = its capacity L in tokens (a
 * multiple of block), so the caches are
 *   k_cache, v_cache [B, Hkv, L, d] (dtype), mu_cache [B, Hkv, L/block, d] fp32,
 * all device memory owned by the caller, who also writes each token's key
 * and value into the caches.  A prompt is processed in chunks
 * (ssa_prefill), then one token at a time (ssa_decode).
 *
 * ssa_cache_block_means: mu_cache[b, c, j] = mean of k_cache[b, c, i] over the
 *   keys i of block j, for blocks block_begin <= j < block_end (the same
 *   means the selection scores against).  Call it for the complete blocks
 *   after a prompt, and for block j once its last key (position
 *   (j+1) * block - 1) is in the cache.  SSA_ERR_SHAPE unless
 *   0 <= block_begin <= block_end <= L / block.
 *
 * ssa_decode: one new token per sequence.  q [B, Hq, d] (dtype) is the token
 *   of sequence b at position pos[b] (device int32 [B]; positions outside
 *   [0, L) are clamped), whose key and value are already at that position of
 *   the caches; it attends causally to keys 0 .. pos[b].
 *     SSA_FULL_ONLY: every key 0 .. pos[b].
 *     SSA_SPARSE_ONLY: its own block (keys up to pos[b]) and the top_k - 1
 *       earlier blocks with the largest q . mu (fp32 scores against
 *       mu_cache, which must hold every complete earlier block), the lower
 *       index winning a tie -- the rule of ssa_select_blocks.  The selection
 *       is written to sel [B, Hq, top_k] (ascending, -1 padded; required).
 *   Writes h [B, Hq, d] (dtype) and, if lse is not NULL, lse [B, Hq] fp32
 *   (natural log).  The workspace is ssa_workspace_size(shape, mode,
 *   SSA_OP_DECODE) bytes (per-part partial outputs).  Other modes return
 *   SSA_ERR_UNSUPPORTED; other errors as for the layer entry points.
 *   The work is the selected keys (sparse) or all pos[b] + 1 keys (full):
 *   each key and value row is read once per query head.
 */
ssa_status_t ssa_cache_block_means(const ssa_shape_t* shape, const void* k_cache, float* mu_cache,
                                   int32_t block_begin, int32_t block_end, void* stream);

/*
 * ssa_prefill: a chunk of `chunk` prompt tokens at positions pos0 ..
 *   pos0 + chunk - 1 of every sequence (chunked prefill), each attending
 *   causally to the cached keys 0 .. its position.  The chunk's keys and
 *   values must already be in the caches; for SSA_SPARSE_ONLY mu_cache must
 *   hold every complete block up to the chunk's end (ssa_cache_block_means
 *   over [0, (pos0 + chunk) / block)).
 *     q [B, Hq, chunk, d], h [B, Hq, chunk, d] (dtype), lse [B, Hq, chunk]
 *     fp32 (natural log, may be NULL), sel [B, Hq, chunk, top_k] int32
 *     (SSA_SPARSE_ONLY: the rows' selection, written; required).
 *   Rows are the layer's rows pos0 .. of the sequence: the same selection
 *   rule and the same kernels as ssa_select_blocks + ssa_attn_fwd (the
 *   sparse stream on key-block buckets, the full stream as the matrix
 *   forward), with the queries offset against the cache.
 *   Requires bf16 (else SSA_ERR_UNSUPPORTED), pos0 and
 *   chunk multiples of block with pos0 + chunk <= seqlen (SSA_ERR_SHAPE),
 *   mode SSA_FULL_ONLY or SSA_SPARSE_ONLY (SSA_ERR_UNSUPPORTED).  Workspace:
 *   ssa_prefill_workspace_size(shape, mode, chunk) bytes (0 on an invalid
 *   request; SSA_FULL_ONLY needs none).
 */
size_t ssa_prefill_workspace_size(const ssa_shape_t* shape, int32_t mode, int32_t chunk);
ssa_status_t ssa_prefill(const ssa_shape_t* shape, int32_t mode, const void* q, int32_t pos0, int32_t chunk,
                         const void* k_cache, const void* v_cache, const float* mu_cache, void* h,
                         float* lse, int32_t* sel, void* ws, size_t ws_bytes, void* stream);
ssa_status_t ssa_decode(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k_cache,
                        const void* v_cache, const float* mu_cache, const int32_t* pos, void* h,
                        float* lse, int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/*
 * Machine probes for measurement harnesses: the two ceilings that the
 * attention kernels' rates are read against.  Not part of the attention
 * method; timed through the hooks above as "probe_mfma" / "probe_copy".
 *
 * ssa_probe_mfma: a dense bf16 matrix-core loop.  `blocks` workgroups of 4
 *   waves (two workgroups per compute unit when blocks >= 2 x the CU count);
 *   every wave runs 4 independent chains of `iters` 32x32x16 bf16 matrix
 *   products (32768 flops each): blocks * 16 * iters * 32768 flops in total.
 *   `sink` (device, blocks * 256 floats, caller-owned) receives the lanes'
 *   accumulator sums so that no product can be dropped; its values mean
 *   nothing.  SSA_ERR_NULL for a null sink, SSA_ERR_SHAPE for blocks < 1 or
 *   iters < 1.
 * ssa_probe_copy: a plain device copy of `bytes` from src to dst (device,
 *   caller-owned, not overlapping): `bytes` read and `bytes` written.
 *   SSA_ERR_NULL for a null pointer, SSA_ERR_SHAPE if bytes is not a multiple
 *   of 16; bytes == 0 returns SSA_OK and launches nothing.
 * Both only enqueue on `stream`; SSA_ERR_HIP reports a launch failure.
 */
ssa_status_t ssa_probe_mfma(float* sink, int32_t blocks, int32_t iters, void* stream);
ssa_status_t ssa_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Two more probes, timed as "probe_atomic" / "probe_lds": the rates that
 * decide how a kernel may combine partial results (atomics) and how much
 * operand traffic it can take from LDS.
 *
 * ssa_probe_atomic: `blocks` workgroups of 256 threads; workgroup w adds 1.0
 *   with fp32 global atomics to every float of 16 KiB tile w % (n_floats /
 *   4096) of `buf` (device, caller-owned, n_floats floats), `iters` times:
 *   blocks * iters * 16 KiB of atomic payload.  Each float of a tile ends up
 *   incremented by iters times the number of workgroups mapped to its tile
 *   (exact for totals below 2^24).  SSA_ERR_NULL for a null buffer,
 *   SSA_ERR_SHAPE unless n_floats is a positive multiple of 4096 (at most
 *   2^20 tiles) and blocks, iters >= 1.
 * ssa_probe_lds: `blocks` workgroups of 4 waves (two per CU); every wave
 *   performs iters * 8 LDS reads, of 16 bytes per lane (mode 0, 1 KiB per
 *   read) or 8 bytes per lane by transposing reads (mode 1, 512 bytes per
 *   read).  Modes 2..9 replay the attention kernels' operand reads (16-byte
 *   row reads, or pairs of transposing reads) on tiles of 256- or 128-byte
 *   rows under several chunk swizzles, for the LDS bank-conflict counter:
 *   2, 3, 4 transposes on 256-byte rows with c ^ (2 (r % 8) + (r / 8) % 2),
 *   c ^ (4 (r % 4) + (r / 4) % 4) and c ^ (r % 16); 5 row reads, 256-byte
 *   rows, the second; 6, 7 row reads and 8, 9 transposes on 128-byte rows
 *   with c ^ (r % 8) and c ^ (4 ((r / 2) % 2) + (r / 4) % 4).  `sink`
 *   (device, blocks * 256 floats) receives meaningless values.
 *   SSA_ERR_NULL / SSA_ERR_SHAPE as above (mode must be 0 .. 9).
 */
ssa_status_t ssa_probe_atomic(float* buf, int64_t n_floats, int32_t blocks, int32_t iters, void* stream);
ssa_status_t ssa_probe_lds(float* sink, int32_t blocks, int32_t iters, int32_t mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
