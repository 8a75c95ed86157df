// C entry points of libssa: argument validation on the host, workspace
// carving, kernel dispatch on the caller's stream, status reporting and the
// optional event timing.  See include/ssa.h for the contract.

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "ssa.h"
#include "internal.h"

namespace ssa {

static thread_local std::string g_last_error;

static ssa_status_t fail(ssa_status_t st, const char* fmt, const char* detail = "") {
  char buf[512];
  snprintf(buf, sizeof(buf), fmt, detail);
  g_last_error = buf;
  return st;
}

// ---------------------------------------------------------------- timing ---
// The library's only process-wide state: the optional event records of the
// measurement hooks, guarded by one mutex.
struct TimingRec {
  int kernel;
  hipEvent_t a, b;
};
static std::mutex g_timing_mu;
static bool g_timing = false;
static std::vector<TimingRec> g_recs;
static const char* kKernelNames[kKernelCount] = {
    "block_mean", "select", "fwd_simt", "fwd_mfma", "loss_reduce",
    "bwd_pre",    "bwd_simt", "bwd_mfma", "convert", "zero", "bucket", "sparse_part", "sparse_merge",
    "bwd_sparse", "bwd_dq", "probe_mfma", "probe_copy", "decode", "dq_merge", "probe_atomic", "probe_lds"};

static thread_local int g_timing_paused = 0;
TimingPause::TimingPause() { ++g_timing_paused; }
TimingPause::~TimingPause() { --g_timing_paused; }

void set_last_error(const char* msg) { g_last_error = msg; }

void timing_begin(int kernel, hipStream_t s) {
  if (g_timing_paused) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing) return;
  TimingRec r{kernel, nullptr, nullptr};
  if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
  (void)hipEventRecord(r.a, s);
  g_recs.push_back(r);
}

void timing_end(int kernel, hipStream_t s) {
  if (g_timing_paused) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing || g_recs.empty()) return;
  TimingRec& r = g_recs.back();
  if (r.kernel == kernel) (void)hipEventRecord(r.b, s);
}

static void timing_clear() {
  for (auto& r : g_recs) {
    if (r.a) (void)hipEventDestroy(r.a);
    if (r.b) (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
}

// ------------------------------------------------------------ validation ---
static ssa_status_t make_dims(const ssa_shape_t* sh, Dims* D) {
  if (!sh) return fail(SSA_ERR_NULL, "shape is NULL%s");
  if (sh->batch < 1 || sh->heads_q < 1 || sh->group < 1 || sh->seqlen < 1 || sh->top_k < 1)
    return fail(SSA_ERR_SHAPE, "batch, heads_q, group, seqlen and top_k must be >= 1%s");
  if (sh->heads_q % sh->group != 0) return fail(SSA_ERR_SHAPE, "group must divide heads_q%s");
  if (sh->dtype != SSA_F32 && sh->dtype != SSA_BF16) return fail(SSA_ERR_UNSUPPORTED, "dtype must be SSA_F32 or SSA_BF16%s");
  if (sh->head_dim != 64 && sh->head_dim != 128) return fail(SSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128%s");
  if (sh->block != 32 && sh->block != 64 && sh->block != 128)
    return fail(SSA_ERR_UNSUPPORTED, "block must be 32, 64 or 128%s");
  if (sh->seqlen % sh->block != 0) return fail(SSA_ERR_SHAPE, "seqlen must be a multiple of block%s");
  const int nb = sh->seqlen / sh->block;
  if (nb > 4096) return fail(SSA_ERR_UNSUPPORTED, "at most 4096 key blocks (seqlen / block) per sequence%s");
  if (sh->top_k > 64 && sh->top_k < nb)
    return fail(SSA_ERR_UNSUPPORTED, "top_k above 64 is supported only when it selects every block%s");
  const int64_t rows = static_cast<int64_t>(sh->batch) * sh->heads_q * sh->seqlen;
  if (rows * sh->head_dim >= (static_cast<int64_t>(1) << 40) || rows / 4 >= (static_cast<int64_t>(1) << 31))
    return fail(SSA_ERR_SHAPE, "layer too large%s");
  if (!(sh->softmax_scale == sh->softmax_scale)) return fail(SSA_ERR_SHAPE, "softmax_scale is NaN%s");
  if (rows * (sh->top_k < nb ? sh->top_k : nb) >= (static_cast<int64_t>(1) << 31))
    return fail(SSA_ERR_SHAPE, "layer too large (rows * min(top_k, N / block) must stay below 2^31)%s");
  D->B = sh->batch;
  D->Hq = sh->heads_q;
  D->G = sh->group;
  D->Hkv = sh->heads_q / sh->group;
  D->N = sh->seqlen;
  D->Nq = sh->seqlen;
  D->q_off = 0;
  D->d = sh->head_dim;
  D->block = sh->block;
  D->nb = nb;
  D->K = sh->top_k;
  D->dtype = sh->dtype;
  D->scale = sh->softmax_scale > 0.f ? sh->softmax_scale : static_cast<float>(1.0 / sqrt(static_cast<double>(sh->head_dim)));
  return SSA_OK;
}

static bool valid_mode(int32_t m) { return m >= kDualFull && m <= kSparseOnly; }

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace carving: a bump allocator over the caller's buffer.
struct Carver {
  char* base;
  size_t used = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += align256(bytes);
    return p;
  }
};

static Buckets carve_buckets(const Dims& D, Carver& c) {
  Buckets b{};
  const int64_t nbk = static_cast<int64_t>(D.B) * D.Hkv * D.nb;
  b.mask = c.take<uint32_t>(bucket_mask_words(D) * sizeof(uint32_t));
  b.count = c.take<int32_t>(nbk * sizeof(int32_t));
  b.offs = c.take<int32_t>((nbk + 1) * sizeof(int32_t));
  b.rows = c.take<int32_t>(bucket_capacity(D) * sizeof(int32_t));
  b.wpos = c.take<int32_t>(bucket_mask_words(D) * sizeof(int32_t));
  return b;
}

struct FwdWs {
  float* row_sq;
  double* loss_sums;
  Buckets bk;                 // sparse-only forward on buckets
  uint16_t* part_o;
  float* part_lse;
};
static FwdWs carve_fwd(const Dims& D, int mode, Carver& c) {
  FwdWs w{};
  if (mode == kDualFull || mode == kDualSparse) {
    w.row_sq = c.take<float>(D.rows() * sizeof(float));
    w.loss_sums = c.take<double>(loss_scratch_bytes());
  }
  if (mode == kSparseOnly && sparse_fwd_supported(D)) {
    w.bk = carve_buckets(D, c);
    // (one spare entry past the buckets' for the part kernel's rows past a bucket's end)
    w.part_o = c.take<uint16_t>((bucket_capacity(D) + 1) * D.d * sizeof(uint16_t));
    w.part_lse = c.take<float>((bucket_capacity(D) + 1) * sizeof(float));
  }
  return w;
}

struct BwdWs {
  // generic path
  float *dk_acc, *dv_acc;
  // MFMA path
  uint16_t *g_full, *g_sparse;
  float *D_full, *D_sparse, *lse2_full, *lse2_sparse;
  uint4* rowv_full;
  uint16_t* dq_part;          // sparse-only: the sparse stream's partial dQ rows (bucket order)
  Buckets bk;                 // sparse stream
  float *dk_part, *dv_part;   // training modes: the sparse stream's fp32 dK / dV
  uint16_t* ds_rows;          // training modes: the sparse stream's dS rows for the dQ kernel
};
static BwdWs carve_bwd(const Dims& D, int mode, Carver& c) {
  BwdWs w{};
  if (bwd_mfma_supported(D)) {
    const bool f = mode != kSparseOnly, sp = mode != kFullOnly;
    if (f) {
      w.g_full = c.take<uint16_t>(D.q_elems() * sizeof(uint16_t));
      w.D_full = c.take<float>(D.rows() * sizeof(float));
      w.lse2_full = c.take<float>(D.rows() * sizeof(float));
      w.rowv_full = c.take<uint4>(D.rows() * sizeof(uint4));
    }
    if (sp) {
      w.g_sparse = c.take<uint16_t>(D.q_elems() * sizeof(uint16_t));
      w.D_sparse = c.take<float>(D.rows() * sizeof(float));
      w.lse2_sparse = c.take<float>(D.rows() * sizeof(float));
      w.bk = carve_buckets(D, c);
    }
    if (f && sp) {
      w.dk_part = c.take<float>(D.kv_elems() * sizeof(float));
      w.dv_part = c.take<float>(D.kv_elems() * sizeof(float));
      w.ds_rows = c.take<uint16_t>(static_cast<size_t>(bucket_capacity(D)) * D.block * sizeof(uint16_t));
    }
    if (sp && !f) w.dq_part = c.take<uint16_t>(static_cast<size_t>(bucket_capacity(D)) * D.d * sizeof(uint16_t));
  } else {
    w.dk_acc = c.take<float>(D.kv_elems() * sizeof(float));
    w.dv_acc = c.take<float>(D.kv_elems() * sizeof(float));
  }
  return w;
}

struct DecodeWs {
  uint32_t* codes;
  float *part_o, *part_ml;
};
static DecodeWs carve_decode(const Dims& D, int mode, Carver& c) {
  const size_t rows = static_cast<size_t>(D.B) * D.Hq;
  const size_t n = rows * decode_parts(D, mode == kSparseOnly);
  DecodeWs w{};
  if (mode == kSparseOnly) w.codes = c.take<uint32_t>(rows * D.nb * sizeof(uint32_t));
  w.part_o = c.take<float>(n * D.d * sizeof(float));
  w.part_ml = c.take<float>(n * 2 * sizeof(float));
  return w;
}

static size_t ws_need(const Dims& D, int mode, int op) {
  Carver c{nullptr};
  if (op == SSA_OP_SELECT) {
    c.take<float>(static_cast<size_t>(D.B) * D.Hkv * D.d * D.nb * sizeof(float));
    c.take<uint16_t>(select_split_bytes(D));
  } else if (op == SSA_OP_FWD) carve_fwd(D, mode, c);
  else if (op == SSA_OP_DECODE) carve_decode(D, mode, c);
  else carve_bwd(D, mode, c);
  return c.used;
}

static ssa_status_t check_ws_bytes(size_t need, void* ws, size_t ws_bytes) {
  if (need == 0) return SSA_OK;
  if (!ws) return fail(SSA_ERR_NULL, "workspace is NULL%s");
  if (ws_bytes < need) return fail(SSA_ERR_WORKSPACE, "workspace too small%s");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SSA_ERR_WORKSPACE, "workspace not 256-byte aligned%s");
  return SSA_OK;
}

static ssa_status_t check_ws(const Dims& D, int mode, int op, void* ws, size_t ws_bytes) {
  return check_ws_bytes(ws_need(D, mode, op), ws, ws_bytes);
}

static ssa_status_t launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return SSA_OK;
}

}  // namespace ssa

using namespace ssa;

extern "C" {

size_t ssa_workspace_size(const ssa_shape_t* shape, int32_t mode, int32_t op) {
  Dims D;
  if (make_dims(shape, &D) != SSA_OK || !valid_mode(mode) || op < SSA_OP_SELECT || op > SSA_OP_DECODE) return 0;
  if (op == SSA_OP_DECODE && mode != kFullOnly && mode != kSparseOnly) return 0;
  return ws_need(D, mode, op);
}

ssa_status_t ssa_select_blocks(const ssa_shape_t* shape, const void* q, const void* k, int32_t* sel,
                               void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Dims D;
  ssa_status_t st = make_dims(shape, &D);
  if (st != SSA_OK) return st;
  if (!q || !k || !sel) return fail(SSA_ERR_NULL, "q, k and sel are required%s");
  if ((st = check_ws(D, 0, SSA_OP_SELECT, ws, ws_bytes)) != SSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c{static_cast<char*>(ws)};
  float* mu = c.take<float>(static_cast<size_t>(D.B) * D.Hkv * D.d * D.nb * sizeof(float));
  uint16_t* split = c.take<uint16_t>(select_split_bytes(D));
  launch_block_mean(D, k, mu, s);
  if ((st = launch_status()) != SSA_OK) return st;
  launch_select(D, q, mu, split, sel, s);
  return launch_status();
}

}  // extern "C"

namespace ssa {
// The forward of ssa_attn_fwd and ssa_attn_fwd_stats (stats null: none).
static ssa_status_t attn_fwd(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k,
                             const void* v, const int32_t* sel, void* h_full, void* h_sparse, float* lse_full,
                             float* lse_sparse, float* delta, float* losses, float* sink_mass, float* entropy,
                             float* head_stats, void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  ssa_status_t st = make_dims(shape, &D);
  if (st != SSA_OK) return st;
  if (!valid_mode(mode)) return fail(SSA_ERR_SHAPE, "unknown mode%s");
  const bool dual = mode == kDualFull || mode == kDualSparse;
  if (!q || !k || !v) return fail(SSA_ERR_NULL, "q, k and v are required%s");
  if (mode != kFullOnly && (!sel || !h_sparse)) return fail(SSA_ERR_NULL, "sel and h_sparse are required%s");
  if (mode != kSparseOnly && !h_full) return fail(SSA_ERR_NULL, "h_full is required%s");
  if (dual && (!delta || !losses)) return fail(SSA_ERR_NULL, "delta and losses are required in dual modes%s");
  if ((st = check_ws(D, mode, SSA_OP_FWD, ws, ws_bytes)) != SSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c{static_cast<char*>(ws)};
  FwdWs w = carve_fwd(D, mode, c);
  if (mode == kSparseOnly && sparse_fwd_supported(D)) {
    launch_buckets(D, sel, w.bk, s);
    if ((st = launch_status()) != SSA_OK) return st;
    SparseFwdArgs p{q, k, v, sel, w.bk.mask, w.bk.offs, w.bk.rows, w.bk.wpos, w.part_o, w.part_lse, h_sparse,
                    lse_sparse};
    launch_sparse_fwd(D, p, s);
    return launch_status();
  }
  FwdArgs a{q, k, v, sel, h_full, h_sparse, lse_full, lse_sparse, delta, w.row_sq, mode, sink_mass, entropy};
  if (mode != kSparseOnly && fwd_mfma_supported(D)) {   // dual and full modes
    const hipError_t e = launch_fwd_mfma(D, a, s);
    if (e != hipSuccess) return fail(SSA_ERR_HIP, "LDS grant of the forward kernel failed: %s", hipGetErrorString(e));
  } else {
    launch_fwd_simt(D, a, s);
  }
  if ((st = launch_status()) != SSA_OK) return st;
  if (dual) {
    launch_loss_reduce(w.row_sq, D.rows(), 1.0 / static_cast<double>(D.q_elems()), w.loss_sums, losses, s);
    if ((st = launch_status()) != SSA_OK) return st;
  }
  if (head_stats) {
    launch_head_means(sink_mass, entropy, static_cast<int64_t>(D.B) * D.Hq, D.N, head_stats, s);
    st = launch_status();
  }
  return st;
}
}  // namespace ssa

extern "C" {

ssa_status_t ssa_attn_fwd(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k,
                          const void* v, const int32_t* sel, void* h_full, void* h_sparse,
                          float* lse_full, float* lse_sparse, float* delta, float* losses, void* ws,
                          size_t ws_bytes, void* stream) {
  g_last_error.clear();
  return attn_fwd(shape, mode, q, k, v, sel, h_full, h_sparse, lse_full, lse_sparse, delta, losses, nullptr,
                  nullptr, nullptr, ws, ws_bytes, stream);
}

ssa_status_t ssa_attn_fwd_stats(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k,
                                const void* v, const int32_t* sel, void* h_full, void* h_sparse,
                                float* lse_full, float* lse_sparse, float* delta, float* losses,
                                float* sink_mass, float* entropy, float* head_stats, void* ws,
                                size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (mode == kSparseOnly) return fail(SSA_ERR_UNSUPPORTED, "the statistics describe the full stream%s");
  if (!sink_mass || !entropy) return fail(SSA_ERR_NULL, "sink_mass and entropy are required%s");
  return attn_fwd(shape, mode, q, k, v, sel, h_full, h_sparse, lse_full, lse_sparse, delta, losses, sink_mass,
                  entropy, head_stats, ws, ws_bytes, stream);
}

ssa_status_t ssa_attn_bwd(const ssa_shape_t* shape, int32_t mode, float w_sparsity, float w_commit,
                          const void* q, const void* k, const void* v, const int32_t* sel,
                          const void* h_full, const void* h_sparse, const float* lse_full,
                          const float* lse_sparse, const void* d_out, void* dq, void* dk, void* dv,
                          void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Dims D;
  ssa_status_t st = make_dims(shape, &D);
  if (st != SSA_OK) return st;
  if (!valid_mode(mode)) return fail(SSA_ERR_SHAPE, "unknown mode%s");
  if (!q || !k || !v || !dq || !dk || !dv) return fail(SSA_ERR_NULL, "q, k, v, dq, dk and dv are required%s");
  if (mode != kFullOnly && (!sel || !h_sparse || !lse_sparse))
    return fail(SSA_ERR_NULL, "sel, h_sparse and lse_sparse are required%s");
  if (mode != kSparseOnly && (!h_full || !lse_full)) return fail(SSA_ERR_NULL, "h_full and lse_full are required%s");
  if (!(w_sparsity == w_sparsity) || !(w_commit == w_commit)) return fail(SSA_ERR_SHAPE, "loss weight is NaN%s");
  if ((st = check_ws(D, mode, SSA_OP_BWD, ws, ws_bytes)) != SSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c{static_cast<char*>(ws)};
  BwdWs w = carve_bwd(D, mode, c);
  if (bwd_mfma_supported(D)) {
    // stream gradients, then the sparse stream on key-block buckets (sparse
    // alone: dK / dV and an fp32 dQ; training modes: dK / dV as fp32 partials
    // and the rows of dS), then the full stream's dK / dV and dQ, each adding
    // the sparse stream's part
    BwdPreArgs p{d_out, h_full, h_sparse, lse_full, lse_sparse, w.g_full, w.g_sparse, w.D_full, w.D_sparse,
                 w.lse2_full, w.lse2_sparse, w.rowv_full, mode};
    launch_bwd_pre(D, p, w_sparsity, w_commit, s);
    if ((st = launch_status()) != SSA_OK) return st;
    if (mode != kFullOnly) {
      launch_buckets(D, sel, w.bk, s);
      if ((st = launch_status()) != SSA_OK) return st;
      SparseBwdArgs sp{q, k, v, w.bk.offs, w.bk.rows, w.g_sparse, w.lse2_sparse, w.D_sparse, w.dq_part,
                       w.ds_rows, w.dk_part, w.dv_part, dk, dv};
      launch_bwd_sparse(D, sp, s);
      if ((st = launch_status()) != SSA_OK) return st;
    }
    if (mode == kSparseOnly) {
      launch_sparse_dq_merge(D, sel, w.bk.mask, w.bk.wpos, w.dq_part, dq, s);
      return launch_status();
    }
    BwdMainArgs m{q, k, v, w.g_full, w.rowv_full, dk, dv, w.dk_part, w.dv_part};
    launch_bwd_mfma(D, m, s);
    if ((st = launch_status()) != SSA_OK) return st;
    BwdDqArgs dqa{q, k, v, w.g_full, w.lse2_full, w.D_full, w.ds_rows ? w.bk.mask : nullptr,
                  w.ds_rows ? w.bk.wpos : nullptr, w.ds_rows, dq};
    launch_bwd_dq(D, dqa, s);
    return launch_status();
  }
  launch_zero_f32(w.dk_acc, D.kv_elems(), s);
  launch_zero_f32(w.dv_acc, D.kv_elems(), s);
  if ((st = launch_status()) != SSA_OK) return st;
  BwdArgs a{q, k, v, sel, h_full, h_sparse, lse_full, lse_sparse, d_out, dq, w.dk_acc, w.dv_acc,
            w_sparsity, w_commit, mode};
  launch_bwd_simt(D, a, s);
  if ((st = launch_status()) != SSA_OK) return st;
  launch_convert(w.dk_acc, dk, D.dtype, D.kv_elems(), s);
  launch_convert(w.dv_acc, dv, D.dtype, D.kv_elems(), s);
  return launch_status();
}

const char* ssa_status_string(int32_t status) {
  switch (status) {
    case SSA_OK: return "ok";
    case SSA_ERR_NULL: return "null pointer";
    case SSA_ERR_SHAPE: return "invalid shape or argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case SSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ssa_last_error(void) { return g_last_error.c_str(); }

ssa_status_t ssa_timing_enable(int32_t enabled) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  timing_clear();
  g_timing = enabled != 0;
  return SSA_OK;
}

ssa_status_t ssa_timing_query(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(SSA_ERR_NULL, "null argument%s");
  int id = -1;
  for (int i = 0; i < kKernelCount; ++i)
    if (strcmp(kernel, kKernelNames[i]) == 0) id = i;
  if (id < 0) return fail(SSA_ERR_SHAPE, "unknown kernel name %s", kernel);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (r.kernel != id || !r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(SSA_ERR_HIP, "event synchronize failed%s");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(SSA_ERR_HIP, "event elapsed time failed%s");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return SSA_OK;
}

}  // extern "C"

namespace ssa {
// Dimensions of a prefill chunk: Nq = chunk query rows at positions pos0 ..
// against the cache of capacity seqlen.
static ssa_status_t prefill_dims(const ssa_shape_t* shape, int32_t mode, int32_t pos0, int32_t chunk, Dims* D) {
  ssa_status_t st = make_dims(shape, D);
  if (st != SSA_OK) return st;
  if (mode != kFullOnly && mode != kSparseOnly)
    return fail(SSA_ERR_UNSUPPORTED, "prefill runs one stream: SSA_FULL_ONLY or SSA_SPARSE_ONLY%s");
  if (D->dtype != 1) return fail(SSA_ERR_UNSUPPORTED, "prefill needs bf16%s");
  if (chunk < 1 || pos0 < 0 || pos0 % D->block != 0 || chunk % D->block != 0 || pos0 + chunk > D->N)
    return fail(SSA_ERR_SHAPE, "need pos0 and chunk multiples of block with pos0 + chunk <= seqlen%s");
  D->Nq = chunk;
  D->q_off = pos0;
  return SSA_OK;
}

// A sparse chunk also selects against the cache's means: the layer forward's
// workspace plus the split of the means.
static size_t prefill_need(const Dims& D, int32_t mode) {
  const size_t fwd = ws_need(D, mode, SSA_OP_FWD);
  return mode == kSparseOnly ? fwd + align256(select_split_bytes(D)) : fwd;
}
}  // namespace ssa

extern "C" {

size_t ssa_prefill_workspace_size(const ssa_shape_t* shape, int32_t mode, int32_t chunk) {
  Dims D;
  if (prefill_dims(shape, mode, 0, chunk, &D) != SSA_OK) {
    g_last_error.clear();
    return 0;
  }
  return prefill_need(D, mode);
}

ssa_status_t ssa_prefill(const ssa_shape_t* shape, int32_t mode, const void* q, int32_t pos0, int32_t chunk,
                         const void* k_cache, const void* v_cache, const float* mu_cache, void* h, float* lse,
                         int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Dims D;
  ssa_status_t st = prefill_dims(shape, mode, pos0, chunk, &D);
  if (st != SSA_OK) return st;
  if (!q || !k_cache || !v_cache || !h) return fail(SSA_ERR_NULL, "q, k_cache, v_cache and h are required%s");
  if (mode == kSparseOnly && (!mu_cache || !sel)) return fail(SSA_ERR_NULL, "mu_cache and sel are required%s");
  if ((st = check_ws_bytes(prefill_need(D, mode), ws, ws_bytes)) != SSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == kFullOnly) {
    FwdArgs a{q, k_cache, v_cache, nullptr, h, nullptr, lse, nullptr, nullptr, nullptr, kFullOnly};
    const hipError_t e = launch_fwd_mfma(D, a, s);
    if (e != hipSuccess) return fail(SSA_ERR_HIP, "LDS grant of the forward kernel failed: %s", hipGetErrorString(e));
    return launch_status();
  }
  Carver c{static_cast<char*>(ws)};
  FwdWs w = carve_fwd(D, mode, c);
  uint16_t* split = c.take<uint16_t>(select_split_bytes(D));
  launch_select(D, q, mu_cache, split, sel, s);
  if ((st = launch_status()) != SSA_OK) return st;
  launch_buckets(D, sel, w.bk, s);
  if ((st = launch_status()) != SSA_OK) return st;
  SparseFwdArgs p{q, k_cache, v_cache, sel, w.bk.mask, w.bk.offs, w.bk.rows, w.bk.wpos, w.part_o, w.part_lse, h, lse};
  launch_sparse_fwd(D, p, s);
  return launch_status();
}

ssa_status_t ssa_cache_block_means(const ssa_shape_t* shape, const void* k_cache, float* mu_cache,
                                   int32_t block_begin, int32_t block_end, void* stream) {
  g_last_error.clear();
  Dims D;
  ssa_status_t st = make_dims(shape, &D);
  if (st != SSA_OK) return st;
  if (!k_cache || !mu_cache) return fail(SSA_ERR_NULL, "k_cache and mu_cache are required%s");
  if (block_begin < 0 || block_end > D.nb || block_begin > block_end)
    return fail(SSA_ERR_SHAPE, "need 0 <= block_begin <= block_end <= seqlen / block%s");
  if (block_begin == block_end) return SSA_OK;
  launch_cache_means(D, k_cache, mu_cache, block_begin, block_end, static_cast<hipStream_t>(stream));
  return launch_status();
}

ssa_status_t ssa_decode(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k_cache,
                        const void* v_cache, const float* mu_cache, const int32_t* pos, void* h, float* lse,
                        int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Dims D;
  ssa_status_t st = make_dims(shape, &D);
  if (st != SSA_OK) return st;
  if (mode != kFullOnly && mode != kSparseOnly)
    return fail(SSA_ERR_UNSUPPORTED, "decode runs one stream: SSA_FULL_ONLY or SSA_SPARSE_ONLY%s");
  if (!q || !k_cache || !v_cache || !pos || !h) return fail(SSA_ERR_NULL, "q, k_cache, v_cache, pos and h are required%s");
  if (mode == kSparseOnly && (!mu_cache || !sel)) return fail(SSA_ERR_NULL, "mu_cache and sel are required%s");
  if ((st = check_ws(D, mode, SSA_OP_DECODE, ws, ws_bytes)) != SSA_OK) return st;
  Carver c{static_cast<char*>(ws)};
  DecodeWs w = carve_decode(D, mode, c);
  DecodeArgs a{q, k_cache, v_cache, mu_cache, pos, mode == kSparseOnly ? sel : nullptr, w.codes, w.part_o, w.part_ml,
               h, lse};
  launch_decode(D, a, static_cast<hipStream_t>(stream));
  return launch_status();
}

ssa_status_t ssa_probe_mfma(float* sink, int32_t blocks, int32_t iters, void* stream) {
  g_last_error.clear();
  if (!sink) return fail(SSA_ERR_NULL, "null sink%s");
  if (blocks < 1 || iters < 1) return fail(SSA_ERR_SHAPE, "blocks and iters must be positive%s");
  launch_probe_mfma(sink, blocks, iters, static_cast<hipStream_t>(stream));
  return launch_status();
}

ssa_status_t ssa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  g_last_error.clear();
  if (!src || !dst) return fail(SSA_ERR_NULL, "null buffer%s");
  if (bytes % 16 != 0) return fail(SSA_ERR_SHAPE, "bytes must be a multiple of 16%s");
  if (bytes == 0) return SSA_OK;
  launch_probe_copy(src, dst, static_cast<int64_t>(bytes), static_cast<hipStream_t>(stream));
  return launch_status();
}

ssa_status_t ssa_probe_atomic(float* buf, int64_t n_floats, int32_t blocks, int32_t iters, void* stream) {
  g_last_error.clear();
  if (!buf) return fail(SSA_ERR_NULL, "null buffer%s");
  if (n_floats < 4096 || n_floats % 4096 != 0 || n_floats / 4096 > (1 << 20))
    return fail(SSA_ERR_SHAPE, "n_floats must be a positive multiple of 4096 (at most 2^20 tiles)%s");
  if (blocks < 1 || iters < 1) return fail(SSA_ERR_SHAPE, "blocks and iters must be positive%s");
  launch_probe_atomic(buf, static_cast<int>(n_floats / 4096), blocks, iters, static_cast<hipStream_t>(stream));
  return launch_status();
}

ssa_status_t ssa_probe_lds(float* sink, int32_t blocks, int32_t iters, int32_t mode, void* stream) {
  g_last_error.clear();
  if (!sink) return fail(SSA_ERR_NULL, "null sink%s");
  if (blocks < 1 || iters < 1 || mode < 0 || mode > 9)
    return fail(SSA_ERR_SHAPE, "blocks and iters must be positive and mode 0 .. 9%s");
  launch_probe_lds(sink, blocks, iters, mode, static_cast<hipStream_t>(stream));
  return launch_status();
}

int32_t ssa_kernel_count(void) { return kKernelCount; }

const char* ssa_kernel_name(int32_t i) { return (i >= 0 && i < kKernelCount) ? kKernelNames[i] : ""; }

}  // extern "C"
