"""GPU parity at the full sizes of the measured layers.

The whole layer runs through the C ABI exactly as the benchmark runs it
(selection, dual forward, backward, same shapes and launch configuration).
The fp64 oracle cannot redo a whole 16K or 64K layer inside a test, so it
checks

* whole (batch, KV head) units of the training layers: every row of the G
  query heads (selection, both streams, lse, delta, dq) and every key of the
  KV head (dk, dv), computed by the oracle on a process pool -- units are
  independent, since dk and dv sum only over their own query heads -- and a
  whole unit of the 64K layer's forward;
* sampled query rows one by one: the selection (rows whose fp64 cutoff
  margin is below 1e-3 are exempt from the equality check, as screening would
  have redrawn them; their GPU selection must still be a valid near-optimal
  one), both streams, their log-sum-exps and delta recomputed by the oracle
  from the GPU's selection of that row, and dq of those rows;
* properties that hold at any size over the whole layer: L_sparsity ==
  L_commit == mean (h_full - h_sparse)^2 of the outputs, 0 <= delta < 1 with
  delta = 1 - exp(lse_sparse - lse_full), and the backward sum rules (over a
  KV head's keys, sum dk = 0 because every softmax Jacobian row sums to zero;
  sum dv = the sum of the group's stream gradients G_full + G_sparse because
  every probability row sums to one).

Inputs are the unscreened seeded draws of the workloads (ssa_inputs).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import ssa_inputs as si
from gpu_cases import MARGIN, TOL, assert_close, check_selection as _check_selection

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_full_ssa_amd  # noqa: F401  (fails loudly when libssa is missing)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ssa():
    import block_sparse_full_ssa_amd as m
    return m


def _sample_rows(rng, N, block, K, n):
    """Positions spanning the whole sequence, including rows that keep every
    earlier block (own block < top_k) and both ends of a block."""
    early = rng.integers(0, min(N, K * block), size=max(2, n // 8))
    edges = np.array([block - 1, block, N - block, N - 1])
    rest = rng.integers(0, N, size=n - early.size - edges.size)
    return np.unique(np.concatenate([early, edges, rest]))


def _check_rows_fwd(name, wl, b, h, t_idx, qf, kf, vf, sel_np, out, dual=True):
    c = h // wl.group
    scale = 1.0 / math.sqrt(wl.head_dim)
    ref = oracle.attend_rows(qf[b, h, t_idx], t_idx, kf[b, c], vf[b, c], sel_np[b, h, t_idx], wl.block, scale)
    dt = wl.dtype
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse") + (("delta",) if dual else ()):
        assert_close(f"{name} {key} b{b} h{h}", out[key][b, h, torch.from_numpy(t_idx)], ref[key], dt)


def _whole_layer_properties(name, out, dtype):
    hf = out["h_full"].double()
    hs = out["h_sparse"].double()
    L = float(((hf - hs) ** 2).mean())
    losses = out["losses"].cpu().numpy()
    assert losses[0] == losses[1]
    assert abs(losses[0] - L) <= 2e-2 * L + 1e-12, (name, losses, L)
    delta = out["delta"]
    assert float(delta.min()) >= 0.0 and float(delta.max()) < 1.0, name
    expect = -torch.expm1(out["lse_sparse"].double() - out["lse_full"].double())
    assert float((delta.double() - expect).abs().max()) <= 1e-5, name


def _unit_check(name, wl, K, mode, b, c, q, k, v, dout, sel_np, out, grads):
    """One whole (batch, KV head) unit against the oracle: the selection of
    every row of its G query heads (margin-aware), both streams, lse and delta
    of every row, dq of every row, and dk / dv of every key of the KV head
    (the oracle on a process pool, from the GPU's selection of each row)."""
    from oracle import parallel

    G, N = wl.group, wl.seqlen
    hs = slice(c * G, (c + 1) * G)
    qf, gf = si.to_f64(q[b, hs]), si.to_f64(dout[b, hs])
    kf, vf = si.to_f64(k[b, c]), si.to_f64(v[b, c])
    mu_c = oracle.block_means(kf[None, None], wl.block)[0, 0]
    t_all = np.arange(N)
    exempt = 0
    for i in range(G):
        exempt += _check_selection(f"{name} unit b{b} c{c} head {i}", qf[i], t_all, mu_c, wl.block, K,
                                   sel_np[b, c * G + i])
    scale = 1.0 / math.sqrt(wl.head_dim)
    res = parallel.unit_step(qf, kf, vf, wl.block, K, scale, mode, dout_u=gf, sel_u=sel_np[b, hs],
                             M=q.numel())
    _say(f"  unit b{b} c{c}: {G} heads x {N} rows, oracle {res['seconds']:.1f} s on {res['workers']} "
         f"processes, selection rows exempt by margin: {exempt}")
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta"):
        assert_close(f"{name} unit {key}", out[key][b, hs], res[key], wl.dtype)
    dq, dk, dv = grads
    assert_close(f"{name} unit dq", dq[b, hs], res["dq"], wl.dtype)
    assert_close(f"{name} unit dk", dk[b, c], res["dk"], wl.dtype)
    assert_close(f"{name} unit dv", dv[b, c], res["dv"], wl.dtype)


# ------------------------------------------------------------- 16K training --

@pytest.mark.parametrize("K, mode, unit", [(16, oracle.DUAL_ACTIVE_SPARSE, (1, 5)),
                                           (4, oracle.DUAL_ACTIVE_FULL, (0, 2)),
                                           (32, oracle.DUAL_ACTIVE_SPARSE, (1, 7))])
def test_train_layer_16k_full_size(K, mode, unit):
    """B=2, 32 query / 8 KV heads, N=16384, d=128, block 64, top_k 4 / 16 /
    32 (the sweep's ends and the default): the benchmark's layer, one training
    step.  One whole (batch, KV head) unit element by element, sampled rows of
    other heads, and the whole layer's properties and sum rules."""
    wl = si.WORKLOADS["train_b2_h32_n16k"]
    _say(f"full-size {wl.name} top_k {K} mode {mode}: draw")
    q, k, v, _ = si.draw_qkv(wl, 0)
    dout = si.draw_dout(wl, 0)
    qd, kd, vd, gd = (x.to("cuda:0") for x in (q, k, v, dout))
    _say("  select / fwd / bwd on the GPU")
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
    dq, dk, dv = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, K, mode, 1.0, 1.0)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    sel_np = sel.cpu().numpy()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    del qd, kd, vd, gd, fwd, sel

    _say("  whole-layer properties")
    _whole_layer_properties(wl.name, out, wl.dtype)
    _unit_check(f"{wl.name} K{K}", wl, K, mode, unit[0], unit[1], q, k, v, dout, sel_np, out, (dq, dk, dv))

    qf, kf, vf, gf = (si.to_f64(x) for x in (q, k, v, dout))
    mu = oracle.block_means(kf, wl.block)
    rng = np.random.default_rng(1)
    exempt = 0
    scale = 1.0 / math.sqrt(wl.head_dim)
    for b, h in ((0, 0), (0, 13), (1, 31)):
        t_idx = _sample_rows(rng, wl.seqlen, wl.block, K, 24)
        _say(f"  rows b{b} h{h}: {t_idx.size}")
        exempt += _check_selection(f"{wl.name} b{b} h{h}", qf[b, h, t_idx], t_idx, mu[b, h // wl.group],
                                   wl.block, K, sel_np[b, h, t_idx])
        _check_rows_fwd(wl.name, wl, b, h, t_idx, qf, kf, vf, sel_np, out)
        ref_dq = oracle.dq_rows(qf, kf, vf, sel_np, wl.block, scale, wl.group, mode, gf, b, h, t_idx)
        assert_close(f"{wl.name} dq b{b} h{h}", dq[b, h, torch.from_numpy(t_idx)], ref_dq, wl.dtype)
    _say(f"  sampled selection rows exempt by margin: {exempt}")

    _say("  backward sum rules")
    g_f, g_s = oracle.stream_grads(mode, gf, out["h_full"].double().numpy(), out["h_sparse"].double().numpy(),
                                   1.0, 1.0)
    G = (g_f + g_s).reshape(wl.batch, wl.hkv, wl.group, wl.seqlen, wl.head_dim).sum(axis=(2, 3))
    dvs = dv.double().numpy()
    dks = dk.double().numpy()
    sum_dv, abs_dv = dvs.sum(axis=2), np.abs(dvs).sum(axis=2)
    sum_dk, abs_dk = dks.sum(axis=2), np.abs(dks).sum(axis=2)
    assert np.all(np.abs(sum_dv - G) <= 2 ** -7 * abs_dv + 1e-6), np.abs(sum_dv - G).max()
    assert np.all(np.abs(sum_dk) <= 2 ** -7 * abs_dk + 1e-6), np.abs(sum_dk).max()


def test_train_layer_16k_sparse_only_unit():
    """The benchmark's layer (B=2, 32 query / 8 KV heads, N=16384, d=128,
    block 64, top_k 16) trained on the sparse stream alone: one whole (batch,
    KV head) unit element by element -- h_sparse and lse_sparse of every row,
    dq of every row and dk / dv of every key, the buckets of the 16K layer
    (thousands of rows per early key block) through the sparse-only backward
    and its dQ merge."""
    wl = si.WORKLOADS["train_b2_h32_n16k"]
    K, mode, b, c = 16, oracle.SPARSE_ONLY, 1, 3
    _say(f"full-size {wl.name} sparse-only unit b{b} c{c}: draw")
    q, k, v, _ = si.draw_qkv(wl, 0)
    dout = si.draw_dout(wl, 0)
    qd, kd, vd, gd = (x.to("cuda:0") for x in (q, k, v, dout))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
    dq, dk, dv = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, K, mode)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    sel_np = sel.cpu().numpy()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    del qd, kd, vd, gd, fwd, sel
    from oracle import parallel

    G = wl.group
    hs = slice(c * G, (c + 1) * G)
    scale = 1.0 / math.sqrt(wl.head_dim)
    res = parallel.unit_step(si.to_f64(q[b, hs]), si.to_f64(k[b, c]), si.to_f64(v[b, c]), wl.block, K, scale, mode,
                             dout_u=si.to_f64(dout[b, hs]), sel_u=sel_np[b, hs], M=q.numel())
    _say(f"  unit b{b} c{c}: oracle {res['seconds']:.1f} s on {res['workers']} processes")
    assert "h_full" not in res and "h_full" not in out
    for key in ("h_sparse", "lse_sparse"):
        assert_close(f"16k sparse-only unit {key}", out[key][b, hs], res[key], wl.dtype)
    assert_close("16k sparse-only unit dq", dq[b, hs], res["dq"], wl.dtype)
    assert_close("16k sparse-only unit dk", dk[b, c], res["dk"], wl.dtype)
    assert_close("16k sparse-only unit dv", dv[b, c], res["dv"], wl.dtype)


def test_train_layer_16k_d64_full_size():
    """The benchmark's training layer with 64-wide heads (B=2, 32 query / 8 KV
    heads, N=16384, d=64, block 64, top_k 16): one training step, one whole
    (batch, KV head) unit element by element and the whole layer's
    properties."""
    wl = si.scaled_down(si.WORKLOADS["train_b2_h32_n16k"], name="train_b2_h32_n16k_d64", head_dim=64)
    K, mode = wl.top_k, oracle.DUAL_ACTIVE_FULL
    _say(f"full-size {wl.name} top_k {K} mode {mode}: draw")
    q, k, v, _ = si.draw_qkv(wl, 0)
    dout = si.draw_dout(wl, 0)
    qd, kd, vd, gd = (x.to("cuda:0") for x in (q, k, v, dout))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
    dq, dk, dv = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, K, mode, 1.0, 1.0)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    sel_np = sel.cpu().numpy()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    del qd, kd, vd, gd, fwd, sel
    _whole_layer_properties(wl.name, out, wl.dtype)
    _unit_check(wl.name, wl, K, mode, 0, 3, q, k, v, dout, sel_np, out, (dq, dk, dv))


# ---------------------------------------------- 4K GQA layer, every unit --

@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE, oracle.FULL_ONLY,
                                  oracle.SPARSE_ONLY])
def test_gqa_n4k_layer_backward_every_unit(mode):
    """B=1, 16 query / 4 KV heads, N=4096, d=128, block 64, top_k 16, unscreened:
    a training step, and every (batch, KV head) unit of the layer element by
    element (all rows' outputs and dq, every key's dk and dv)."""
    _gqa_n4k_every_unit(si.WORKLOADS["gqa_n4k_fwd"], mode)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE, oracle.FULL_ONLY,
                                  oracle.SPARSE_ONLY])
def test_gqa_n4k_d64_layer_backward_every_unit(mode):
    """The same layer with 64-wide heads and 128-key blocks at top_k 8 (the
    matrix kernels' d = 64 variants, four key halves per block in the bucket
    kernels): every unit element by element."""
    wl = si.scaled_down(si.WORKLOADS["gqa_n4k_fwd"], name="gqa_n4k_d64_b128", head_dim=64, block=128, top_k=8)
    _gqa_n4k_every_unit(wl, mode)


def _gqa_n4k_every_unit(wl, mode):
    K = wl.top_k
    _say(f"{wl.name} whole-layer backward mode {mode}")
    q, k, v, _ = si.draw_qkv(wl, 0)
    dout = si.draw_dout(wl, 0)
    qd, kd, vd, gd = (x.to("cuda:0") for x in (q, k, v, dout))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
    grads = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, K, mode, 0.7, 1.3)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    grads = tuple(x.cpu() for x in grads)
    sel_np = sel.cpu().numpy()
    dual = mode in (oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE)
    if dual:
        _whole_layer_properties(wl.name, out, wl.dtype)
    from oracle import parallel

    scale = 1.0 / math.sqrt(wl.head_dim)
    G = wl.group
    for c in range(wl.hkv):
        hs = slice(c * G, (c + 1) * G)
        qf, gf = si.to_f64(q[0, hs]), si.to_f64(dout[0, hs])
        kf, vf = si.to_f64(k[0, c]), si.to_f64(v[0, c])
        mu_c = oracle.block_means(kf[None, None], wl.block)[0, 0]
        for i in range(G):
            _check_selection(f"4k c{c} head {i}", qf[i], np.arange(wl.seqlen), mu_c, wl.block, K,
                             sel_np[0, c * G + i])
        res = parallel.unit_step(qf, kf, vf, wl.block, K, scale, mode, dout_u=gf, sel_u=sel_np[0, hs],
                                 w_sparsity=0.7, w_commit=1.3, M=q.numel())
        for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta"):
            if key in res:
                assert_close(f"4k c{c} {key}", out[key][0, hs], res[key], wl.dtype)
        assert_close(f"4k c{c} dq", grads[0][0, hs], res["dq"], wl.dtype)
        assert_close(f"4k c{c} dk", grads[1][0, c], res["dk"], wl.dtype)
        assert_close(f"4k c{c} dv", grads[2][0, c], res["dv"], wl.dtype)


# ----------------------------------------------------- selection, many blocks --

@pytest.mark.parametrize("block, nb, top_k, d", [(32, 1100, 8, 64), (64, 4096, 16, 128)])
def test_select_many_blocks(block, nb, top_k, d):
    """1100 and 4096 key blocks (the supported maximum): five and sixteen
    chunks of candidates with carried winners; sampled rows against the
    oracle, margin-aware as above."""
    wl = si.scaled_down(si.WORKLOADS["gqa_n4k_fwd"], seqlen=block * nb, hq=1, hkv=1, block=block,
                        top_k=top_k, head_dim=d)
    _say(f"select nb {nb} block {block} d {d}: draw")
    q, k, _, _ = si.draw_qkv(wl, 0)
    sel = ssa().ssa_select_blocks(q.to("cuda:0"), k.to("cuda:0"), block, top_k).cpu().numpy()
    torch.cuda.synchronize()
    qf, kf = si.to_f64(q), si.to_f64(k)
    mu = oracle.block_means(kf, block)
    t_idx = _sample_rows(np.random.default_rng(2), wl.seqlen, block, top_k, 64)
    exempt = _check_selection(f"nb {nb}", qf[0, 0, t_idx], t_idx, mu[0, 0], block, top_k, sel[0, 0, t_idx])
    _say(f"  rows {t_idx.size}, exempt by margin: {exempt}")
    # every row: ascending, own block last among the kept, padded with -1
    i = np.arange(wl.seqlen) // block
    kept = (sel[0, 0] >= 0).sum(axis=1)
    assert np.all(kept == np.minimum(top_k, i + 1))
    last = sel[0, 0][np.arange(wl.seqlen), kept - 1]
    assert np.all(last == i)


# ---------------------------------------- sparse-only forward, > 64 blocks kept --

def test_sparse_only_fwd_many_blocks_kept():
    """top_k 128 of 128 blocks (top_k above 64 is accepted only when it keeps
    every block): more than 64 partials per row take the merge's serial path;
    sampled rows against the oracle for the GPU's selection."""
    wl = si.scaled_down(si.WORKLOADS["gqa_n4k_fwd"], seqlen=8192, hq=2, hkv=1, top_k=128)
    K = wl.top_k
    _say("sparse-only forward, top_k 128 of 128 blocks: draw")
    q, k, v, _ = si.draw_qkv(wl, 0)
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, oracle.SPARSE_ONLY)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    sel_np = sel.cpu().numpy()
    qf, kf, vf = (si.to_f64(x) for x in (q, k, v))
    scale = 1.0 / math.sqrt(wl.head_dim)
    for h in range(wl.hq):
        t_idx = _sample_rows(np.random.default_rng(3 + h), wl.seqlen, wl.block, K, 48)
        ref = oracle.attend_rows(qf[0, h, t_idx], t_idx, kf[0, 0], vf[0, 0], sel_np[0, h, t_idx], wl.block, scale)
        for key in ("h_sparse", "lse_sparse"):
            assert_close(f"top_k 128 {key} h{h}", out[key][0, h, torch.from_numpy(t_idx)], ref[key], wl.dtype)


# ----------------------------------------------------------- 64K with sinks --

def test_long_layer_64k_sinks_full_size():
    """B=1, 16 query / 4 KV heads, N=65536, d=128, block 64, top_k 32, four
    planted sink keys: dual forward with the sparse stream active."""
    wl = si.WORKLOADS["long_n64k_sinks"]
    K, mode = wl.top_k, oracle.DUAL_ACTIVE_SPARSE
    _say(f"full-size {wl.name}: draw")
    q, k, v, _ = si.draw_qkv(wl, 0)
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
    torch.cuda.synchronize()
    out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
    sel_np = sel.cpu().numpy()
    del qd, kd, vd, fwd, sel
    _whole_layer_properties(wl.name, out, wl.dtype)
    # the sink block is kept by a large share of the queries
    share = float((sel_np[..., 0] == 0).mean())
    _say(f"  rows keeping block 0: {share:.3f}")
    assert share > 0.3

    qf, kf, vf = (si.to_f64(x) for x in (q, k, v))
    mu = oracle.block_means(kf, wl.block)
    rng = np.random.default_rng(2)
    for b, h in ((0, 0), (0, 11)):
        t_idx = _sample_rows(rng, wl.seqlen, wl.block, K, 16)
        _say(f"  rows b{b} h{h}: {t_idx.size}")
        _check_selection(f"{wl.name} b{b} h{h}", qf[b, h, t_idx], t_idx, mu[b, h // wl.group], wl.block, K,
                         sel_np[b, h, t_idx])
        _check_rows_fwd(wl.name, wl, b, h, t_idx, qf, kf, vf, sel_np, out)

    # one whole (batch, KV head) unit: every row of its G query heads
    from oracle import parallel

    c = 2
    G = wl.group
    hs = slice(c * G, (c + 1) * G)
    for i in range(G):
        _check_selection(f"{wl.name} unit c{c} head {i}", qf[0, c * G + i], np.arange(wl.seqlen), mu[0, c],
                         wl.block, K, sel_np[0, c * G + i])
    res = parallel.unit_step(qf[0, hs], kf[0, c], vf[0, c], wl.block, K, 1.0 / math.sqrt(wl.head_dim), mode,
                             sel_u=sel_np[0, hs], backward=False)
    _say(f"  unit b0 c{c}: {G} heads x {wl.seqlen} rows, oracle {res['seconds']:.1f} s on {res['workers']} processes")
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta"):
        assert_close(f"{wl.name} unit {key}", out[key][0, hs], res[key], wl.dtype)


def test_long_layer_64k_sink_stats_full_size():
    """The 64K layer with planted sinks, full stream with its diagnostics:
    sink-block mass and entropy on sampled rows against the oracle, and over
    the whole layer 0 <= sink <= 1 (= 1 inside the first block),
    0 <= entropy <= ln(t + 1), head means = the means of the rows."""
    wl = si.WORKLOADS["long_n64k_sinks"]
    _say(f"full-size {wl.name}: full stream with statistics")
    q, k, v, _ = si.draw_qkv(wl, 0)
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, None, wl.block, wl.top_k, oracle.FULL_ONLY, stats=True)
    torch.cuda.synchronize()
    sink, ent, hs = (fwd[key].double().cpu() for key in ("sink_mass", "entropy", "head_stats"))
    del qd, kd, vd, fwd
    t = torch.arange(wl.seqlen, dtype=torch.float64)
    assert float(sink.min()) >= 0.0 and float(sink.max()) <= 1.0 + 1e-6
    assert float((sink[..., :wl.block] - 1.0).abs().max()) <= 1e-6
    assert float(ent.min()) >= -1e-5 and bool((ent <= torch.log(t + 1) + 1e-4).all())
    assert float((hs[..., 0] - sink.mean(dim=2)).abs().max()) <= 1e-6
    assert float((hs[..., 1] - ent.mean(dim=2)).abs().max()) <= 1e-5 * float(ent.abs().max())
    _say(f"  mean sink mass {float(sink.mean()):.4f}, mean entropy {float(ent.mean()):.4f}")

    qf, kf = si.to_f64(q), si.to_f64(k)
    rng = np.random.default_rng(3)
    scale = 1.0 / math.sqrt(wl.head_dim)
    for b, h in ((0, 1), (0, 14)):
        t_idx = _sample_rows(rng, wl.seqlen, wl.block, wl.top_k, 16)
        _say(f"  rows b{b} h{h}: {t_idx.size}")
        rs, re = oracle.stats_rows(qf[b, h, t_idx], t_idx, kf[b, h // wl.group], wl.block, scale)
        idx = torch.from_numpy(t_idx)
        assert float(np.abs(sink[b, h, idx].numpy() - rs).max()) <= 1e-4 + 1e-4 * float(np.abs(rs).max())
        assert np.all(np.abs(ent[b, h, idx].numpy() - re) <= 1e-4 + 1e-4 * np.abs(re))


# ----------------------------------------------------------- 4-layer slice --

def test_multilayer_slice_full_size():
    """Four layers of B=4, 32 query / 8 KV heads, N=8192, d=128, block 64,
    top_k 16, each with its own inputs: forward layer 1 to 4, then backward
    layer 4 to 1, one active stream for the whole step; sampled rows of every
    layer against the oracle."""
    wl = si.WORKLOADS["multilayer_b4_n8k_l4"]
    K = wl.top_k
    mode = oracle.DUAL_ACTIVE_FULL if si.draw_modes(0, 1)[0] == 0 else oracle.DUAL_ACTIVE_SPARSE
    scale = 1.0 / math.sqrt(wl.head_dim)
    saved = []
    for layer in range(wl.layers):
        _say(f"full-size {wl.name}: forward layer {layer + 1}")
        q, k, v, _ = si.draw_qkv(wl, 0, layer)
        qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
        sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
        fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, mode)
        saved.append((q, k, v, qd, kd, vd, sel, fwd))
    grads = [None] * wl.layers
    for layer in reversed(range(wl.layers)):
        q, k, v, qd, kd, vd, sel, fwd = saved[layer]
        gd = si.draw_dout(wl, 0, layer).to("cuda:0")
        grads[layer] = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, K, mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for layer in range(wl.layers):
        q, k, v, qd, kd, vd, sel, fwd = saved[layer]
        out = {key: val.cpu() for key, val in fwd.items() if not key.startswith("_")}
        _whole_layer_properties(f"{wl.name} layer {layer + 1}", out, wl.dtype)
        sel_np = sel.cpu().numpy()
        qf, kf, vf = (si.to_f64(x) for x in (q, k, v))
        gf = si.to_f64(si.draw_dout(wl, 0, layer))
        b, h = layer % wl.batch, (7 * layer) % wl.hq
        t_idx = _sample_rows(rng, wl.seqlen, wl.block, K, 12)
        _say(f"  layer {layer + 1} rows b{b} h{h}: {t_idx.size}")
        _check_rows_fwd(f"{wl.name} layer {layer + 1}", wl, b, h, t_idx, qf, kf, vf, sel_np, out)
        ref_dq = oracle.dq_rows(qf, kf, vf, sel_np, wl.block, scale, wl.group, mode, gf, b, h, t_idx)
        g_cpu = tuple(x.cpu() for x in grads[layer])
        assert_close(f"{wl.name} layer {layer + 1} dq", g_cpu[0][b, h, torch.from_numpy(t_idx)], ref_dq, wl.dtype)
        del qf, kf, vf, gf
        # one whole unit of every layer: dk / dv of all its keys, dq of all its rows
        ub, uc = (layer + 1) % wl.batch, (3 * layer + 1) % wl.hkv
        _unit_check(f"{wl.name} layer {layer + 1}", wl, K, mode, ub, uc, q, k, v, si.draw_dout(wl, 0, layer),
                    sel_np, out, g_cpu)
