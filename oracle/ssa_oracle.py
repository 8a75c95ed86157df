"""CPU oracle for SSA dual-stream block-sparse attention (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path.

It writes out, plainly and slowly, what one attention layer of SSA computes
(the paper "SSA: Sparse Sparse Attention by Aligning Full and Sparse Attention
Outputs in Feature Space", arXiv 2511.20102):

* the full-attention stream (every causal key) and the block-sparse stream
  (only the keys of the selected key blocks), which share the same logits
  (Sintesi Tecnica, section 2 'Meccanismo Core'; Resume technique, section 2);
* the discarded attention mass delta(t): the full-attention probability that
  falls on keys the sparse stream leaves out (Sintesi Tecnica, section 2,
  'Allineamento Bidirezionale', item 1; the linear error bound of section 1);
* the alignment losses L_sparsity (h_full pulled toward a stop-gradient
  h_sparse) and L_commit (h_sparse pulled toward a stop-gradient h_full),
  which form L_align in the total objective of section 2;
* the backward pass of both streams with the upstream gradient routed to the
  active stream only, since the counterpart output is used for alignment and
  is not passed to later layers (section 2, 'Allineamento Bidirezionale').

The pages leave the block-selection rule open; it is fixed here as: score
each earlier key block j of query t by q_t . mean(k over block j), always keep
the query's own block, and take the remaining top_k - 1 blocks by score, the
lower block index winning a tie.  Inference 'identical to MoBA' (section 4,
'Efficienza') is the reading that the selection is per query and per block.

Conventions (readings where the pages are silent):
  * logits z[t, i] = scale * q_t . k_i for keys i <= t (causal);
  * query head h reads KV head h // group (grouped-query attention);
  * losses are means over all B*Hq*N*d output elements of one layer;
  * the sparse support A_t is every causal key i <= t whose block is
    selected; inside the own block the mask is token-causal.

Everything here is float64; bf16 or fp32 inputs convert to float64 exactly.
Parity is pinned by the not-gpu tests (brute force, SDPA, closed forms, the
Appendix-style identity h_full - h_sparse = delta (h_u - h_sparse), finite
differences and torch autograd).
"""
from __future__ import annotations

import numpy as np

# Stream-routing modes of one training step, mirroring the C interface.
DUAL_ACTIVE_FULL = 0    # both streams; the full output goes to the next layer
DUAL_ACTIVE_SPARSE = 1  # both streams; the sparse output goes to the next layer
FULL_ONLY = 2           # full attention alone
SPARSE_ONLY = 3         # block-sparse attention alone (inference)

_ROW_CHUNK = 512


# ---------------------------------------------------------------------------
# Block selection
# ---------------------------------------------------------------------------

def block_means(k: np.ndarray, block: int) -> np.ndarray:
    """mu[b, c, j, :] = mean of k[b, c, i, :] over the keys i of block j.

    k: [B, Hkv, N, d] -> [B, Hkv, N // block, d].  Blocks are consecutive,
    equal-sized runs of keys (block-sparse attention, Sintesi Tecnica s.2).
    """
    B, H, N, d = k.shape
    nb = N // block
    return k.reshape(B, H, nb, block, d).mean(axis=3)


def select_rows(q_rows: np.ndarray, t_idx: np.ndarray, mu_c: np.ndarray,
                block: int, top_k: int):
    """Selected key blocks of some query rows of one head.

    q_rows: [R, d] queries at positions t_idx [R]; mu_c: [nb, d] block means
    of the head's KV head.  Returns (sel [R, top_k] int32, ascending block
    indices padded with -1; margin [R] float64).

    For row t with own block i_t = t // block the candidates are the earlier
    blocks j < i_t with score sigma_j = q_t . mu_j.  They are ranked by
    descending score, equal scores by ascending j (a stable sort of -sigma),
    the first min(top_k - 1, i_t) are kept and i_t is added.  ``margin`` is
    the score gap across the cutoff, sigma of the last kept minus sigma of the
    first dropped candidate, or +inf when nothing is dropped.
    """
    R = q_rows.shape[0]
    sel = np.full((R, top_k), -1, dtype=np.int32)
    margin = np.full(R, np.inf)
    own = t_idx // block
    for i in np.unique(own):
        rows = np.nonzero(own == i)[0]
        keep = min(top_k - 1, int(i))
        chosen = np.empty((rows.size, 0), dtype=np.int64)
        if keep > 0:
            sigma = q_rows[rows] @ mu_c[:i].T                 # [r, i]
            order = np.argsort(-sigma, axis=1, kind="stable")
            chosen = order[:, :keep]
            if i > keep:
                ranked = np.take_along_axis(sigma, order, axis=1)
                margin[rows] = ranked[:, keep - 1] - ranked[:, keep]
        full = np.concatenate([chosen, np.full((rows.size, 1), i)], axis=1)
        full.sort(axis=1)
        sel[rows, :full.shape[1]] = full
    return sel, margin


def select_blocks(q: np.ndarray, k: np.ndarray, block: int, top_k: int, group: int):
    """Per (batch, query head, token) top-k key blocks.

    q: [B, Hq, N, d], k: [B, Hkv, N, d].  Returns sel [B, Hq, N, top_k] int32
    and the cutoff margin [B, Hq, N].
    """
    B, Hq, N, d = q.shape
    mu = block_means(k, block)
    t_idx = np.arange(N)
    sel = np.empty((B, Hq, N, top_k), dtype=np.int32)
    margin = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            sel[b, h], margin[b, h] = select_rows(q[b, h], t_idx, mu[b, h // group], block, top_k)
    return sel, margin


# ---------------------------------------------------------------------------
# The two attention streams
# ---------------------------------------------------------------------------

def _support(sel_rows: np.ndarray, t_idx: np.ndarray, n_keys: int, block: int):
    """Boolean masks [R, n_keys]: causal (i <= t) and sparse support A_t."""
    keys = np.arange(n_keys)
    causal = keys[None, :] <= t_idx[:, None]
    nb = (n_keys + block - 1) // block
    chosen = np.zeros((sel_rows.shape[0], nb + 1), dtype=bool)
    rows = np.repeat(np.arange(sel_rows.shape[0]), sel_rows.shape[1])
    cols = sel_rows.reshape(-1).astype(np.int64)
    cols = np.where(cols < 0, nb, cols)          # padding lands in a spare column
    chosen[rows, cols] = True
    in_sparse = chosen[:, keys // block]
    return causal, causal & in_sparse


def _softmax_rows(z: np.ndarray, mask: np.ndarray):
    """Softmax of z over the True entries of each row; returns (p, lse)."""
    zm = np.where(mask, z, -np.inf)
    m = zm.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(zm - m), 0.0)
    s = e.sum(axis=1, keepdims=True)
    return e / s, (m + np.log(s))[:, 0]


def attend_rows(q_rows, t_idx, k_c, v_c, sel_rows, block, scale,
                want_full=True, want_sparse=True):
    """Both streams for some query rows of one head.

    q_rows [R, d] at positions t_idx; k_c, v_c [N, d] of the KV head;
    sel_rows [R, top_k].  Returns a dict with h_full, h_sparse [R, d],
    lse_full, lse_sparse, delta [R] (missing streams are omitted).
    """
    n_keys = int(t_idx.max()) + 1
    z = scale * (q_rows @ k_c[:n_keys].T)                   # [R, n_keys]
    causal, A = _support(sel_rows if sel_rows is not None else
                         np.zeros((len(t_idx), 0), np.int32), t_idx, n_keys, block)
    out = {}
    if want_full:
        p_f, lse_f = _softmax_rows(z, causal)
        out["h_full"] = p_f @ v_c[:n_keys]
        out["lse_full"] = lse_f
    if want_sparse:
        p_s, lse_s = _softmax_rows(z, A)
        out["h_sparse"] = p_s @ v_c[:n_keys]
        out["lse_sparse"] = lse_s
    if want_full and want_sparse:
        # delta(t): full-attention mass on the causal keys outside A_t
        out["delta"] = np.where(causal & ~A, p_f, 0.0).sum(axis=1)
    return out


def forward(q, k, v, sel, block, scale, group, mode=DUAL_ACTIVE_FULL):
    """Forward of one SSA layer.

    q [B,Hq,N,d]; k, v [B,Hkv,N,d]; sel [B,Hq,N,top_k].  Dual modes return
    h_full, h_sparse, lse_full, lse_sparse, delta and the two losses;
    FULL_ONLY / SPARSE_ONLY return that stream's output and lse.
    """
    B, Hq, N, d = q.shape
    want_full = mode != SPARSE_ONLY
    want_sparse = mode != FULL_ONLY
    res = {}
    if want_full:
        res["h_full"] = np.zeros((B, Hq, N, d))
        res["lse_full"] = np.zeros((B, Hq, N))
    if want_sparse:
        res["h_sparse"] = np.zeros((B, Hq, N, d))
        res["lse_sparse"] = np.zeros((B, Hq, N))
    if want_full and want_sparse:
        res["delta"] = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            c = h // group
            for t0 in range(0, N, _ROW_CHUNK):
                t_idx = np.arange(t0, min(N, t0 + _ROW_CHUNK))
                o = attend_rows(q[b, h, t_idx], t_idx, k[b, c], v[b, c],
                                None if sel is None else sel[b, h, t_idx],
                                block, scale, want_full, want_sparse)
                for key, val in o.items():
                    res[key][b, h, t_idx] = val
    if want_full and want_sparse:
        L = alignment_loss(res["h_full"], res["h_sparse"])
        res["L_sparsity"] = L
        res["L_commit"] = L
    return res


def alignment_loss(h_full, h_sparse):
    """Mean squared distance of the two outputs over all B*Hq*N*d elements.

    L_sparsity and L_commit have this same value; they differ only in which
    side is held fixed (stop-gradient) when differentiating.
    """
    diff = h_full - h_sparse
    return float((diff * diff).sum() / diff.size)


# ---------------------------------------------------------------------------
# Diagnostics of the full stream
# ---------------------------------------------------------------------------

def full_stats(q, k, block, scale, group):
    """Per-row statistics of the full-attention distribution p_f(t, .).

    The pages measure two properties of the attention distribution without
    defining a statistic for either; the readings fixed here are:
      * sink mass: the total p_f(t, i) on the keys of the first key block
        (i < block), the sink area at the start of the sequence whose
        over-allocation of attention the English abstract ties to poor
        length extrapolation (its last sentence);
      * sparsity: the entropy -sum_i p_f(t, i) ln p_f(t, i) in nats over the
        causal keys; lower means more concentrated ("intrinsically sparser")
        attention, which SSA aims for (Sintesi Tecnica, section 5,
        'Sparsita Intrinseca').
    Returns (sink_mass, entropy), both [B, Hq, N], and head_means [B, Hq, 2]
    (the mean over the N rows of each).
    """
    B, Hq, N, _ = q.shape
    sink = np.zeros((B, Hq, N))
    ent = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            c = h // group
            for t0 in range(0, N, _ROW_CHUNK):
                t_idx = np.arange(t0, min(N, t0 + _ROW_CHUNK))
                sink[b, h, t_idx], ent[b, h, t_idx] = stats_rows(q[b, h, t_idx], t_idx, k[b, c], block, scale)
    means = np.stack([sink.mean(axis=2), ent.mean(axis=2)], axis=2)
    return sink, ent, means


def stats_rows(q_rows, t_idx, k_c, block, scale):
    """(sink_mass, entropy) [R] of full_stats for some query rows of one head
    (q_rows [R, d] at positions t_idx; k_c [N, d] of its KV head)."""
    n_keys = int(t_idx.max()) + 1
    z = scale * (q_rows @ k_c[:n_keys].T)
    causal = np.arange(n_keys)[None, :] <= t_idx[:, None]
    p, _ = _softmax_rows(z, causal)
    sink = p[:, :min(block, n_keys)].sum(axis=1)
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return sink, -plogp.sum(axis=1)


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def stream_grads(mode, dout, h_full, h_sparse, w_sparsity, w_commit, M=None):
    """Gradients that reach the two outputs, (G_full, G_sparse).

    The upstream gradient ``dout`` reaches only the active stream.  In the
    dual modes the full output also receives the gradient of
    w_sparsity * L_sparsity (h_sparse held fixed) and the sparse output that
    of w_commit * L_commit (h_full held fixed); with L = sum(diff^2) / M that
    is +-(2 / M) * (h_full - h_sparse).  Single-stream modes have no
    counterpart and no alignment term.  ``M`` defaults to the element count
    of the arrays (pass the whole layer's count when these are a row sample).
    """
    if mode == FULL_ONLY:
        return dout, None
    if mode == SPARSE_ONLY:
        return None, dout
    if M is None:
        M = h_full.size
    diff = h_full - h_sparse
    g_f = w_sparsity * (2.0 / M) * diff
    g_s = w_commit * (2.0 / M) * (-diff)
    if dout is not None:
        if mode == DUAL_ACTIVE_FULL:
            g_f = g_f + dout
        else:
            g_s = g_s + dout
    return g_f, g_s


def backward(q, k, v, sel, block, scale, group, mode, dout,
             w_sparsity=1.0, w_commit=1.0, fwd=None):
    """dq [B,Hq,N,d], dk and dv [B,Hkv,N,d] of one SSA layer.

    Differentiates <G_full, h_full> + <G_sparse, h_sparse> with the stream
    gradients of ``stream_grads`` held fixed.  For each stream X with
    probabilities p^X:  D_t = G_t . h_t,  dZ[t,i] = p[t,i] (G_t . v_i - D_t),
    dq_t = scale sum_i dZ[t,i] k_i,  dk_i = scale sum_t dZ[t,i] q_t,
    dv_i = sum_t p[t,i] G_t, with dk/dv summed over the query heads sharing a
    KV head.  The selection is piecewise constant, so no gradient flows
    through the block scores.  ``dout`` may be None (no upstream gradient).
    """
    if fwd is None:
        fwd = forward(q, k, v, sel, block, scale, group, mode)
    g_f, g_s = stream_grads(mode, dout, fwd.get("h_full"), fwd.get("h_sparse"),
                            w_sparsity, w_commit)
    B, Hq, N, d = q.shape
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            c = h // group
            for t0 in range(0, N, _ROW_CHUNK):
                t_idx = np.arange(t0, min(N, t0 + _ROW_CHUNK))
                _bwd_rows(q[b, h], k[b, c], v[b, c], t_idx,
                          None if sel is None else sel[b, h, t_idx], block, scale,
                          _rows_of(g_f, b, h, t_idx), _rows_of(g_s, b, h, t_idx),
                          _rows_of(fwd.get("h_full"), b, h, t_idx),
                          _rows_of(fwd.get("h_sparse"), b, h, t_idx),
                          dq[b, h], dk[b, c], dv[b, c])
    return dq, dk, dv


def _rows_of(x, b, h, t_idx):
    return None if x is None else x[b, h, t_idx]


def _bwd_rows(q_h, k_c, v_c, t_idx, sel_rows, block, scale, g_f, g_s, h_f, h_s,
              dq_h, dk_c, dv_c):
    """Adds the contribution of query rows t_idx of one head to dq, dk, dv."""
    n_keys = int(t_idx.max()) + 1
    q_rows = q_h[t_idx]
    kk, vv = k_c[:n_keys], v_c[:n_keys]
    z = scale * (q_rows @ kk.T)
    causal, A = _support(sel_rows if sel_rows is not None else
                         np.zeros((len(t_idx), 0), np.int32), t_idx, n_keys, block)
    dz = np.zeros_like(z)
    for g, hx, mask in ((g_f, h_f, causal), (g_s, h_s, A)):
        if g is None:
            continue
        p, _ = _softmax_rows(z, mask)
        D = (g * hx).sum(axis=1, keepdims=True)
        dz += p * (g @ vv.T - D)
        dv_c[:n_keys] += p.T @ g
    dq_h[t_idx] += scale * (dz @ kk)
    dk_c[:n_keys] += scale * (dz.T @ q_rows)


def _row_stream_grads(q, k, v, sel, block, scale, group, mode, dout, b, h, t_idx,
                      w_sparsity, w_commit):
    """Outputs and stream gradients of some rows of one head (layer-wide M)."""
    c = h // group
    o = attend_rows(q[b, h, t_idx], t_idx, k[b, c], v[b, c],
                    None if sel is None else sel[b, h, t_idx], block, scale,
                    mode != SPARSE_ONLY, mode != FULL_ONLY)
    hf, hs = o.get("h_full"), o.get("h_sparse")
    g_f, g_s = stream_grads(mode, None if dout is None else dout[b, h, t_idx],
                            hf, hs, w_sparsity, w_commit, M=q.size)
    return hf, hs, g_f, g_s


def dq_rows(q, k, v, sel, block, scale, group, mode, dout, b, h, t_idx,
            w_sparsity=1.0, w_commit=1.0):
    """dq[b, h, t_idx] computed from those rows alone (for large layers)."""
    hf, hs, g_f, g_s = _row_stream_grads(q, k, v, sel, block, scale, group, mode,
                                         dout, b, h, t_idx, w_sparsity, w_commit)
    N, d = q.shape[2], q.shape[3]
    c = h // group
    dq_h, dk_c, dv_c = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    _bwd_rows(q[b, h], k[b, c], v[b, c], t_idx,
              None if sel is None else sel[b, h, t_idx], block, scale,
              g_f, g_s, hf, hs, dq_h, dk_c, dv_c)
    return dq_h[t_idx]


def dkdv_tail(q, k, v, sel, block, scale, group, mode, dout, b, c, i0,
              w_sparsity=1.0, w_commit=1.0):
    """dk, dv of KV head c for the keys i0..N-1 (for large layers).

    Only queries t >= i0 see these keys, so the rows i0..N-1 of the query
    heads of the group give their whole gradient.
    """
    N, d = q.shape[2], q.shape[3]
    dq_h, dk_c, dv_c = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    t_idx = np.arange(i0, N)
    for h in range(c * group, (c + 1) * group):
        hf, hs, g_f, g_s = _row_stream_grads(q, k, v, sel, block, scale, group, mode,
                                             dout, b, h, t_idx, w_sparsity, w_commit)
        _bwd_rows(q[b, h], k[b, c], v[b, c], t_idx,
                  None if sel is None else sel[b, h, t_idx], block, scale,
                  g_f, g_s, hf, hs, dq_h, dk_c, dv_c)
    return dk_c[i0:], dv_c[i0:]
