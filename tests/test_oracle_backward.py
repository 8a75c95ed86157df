"""Pins of the oracle's backward pass (CPU).

References: torch float64 autograd through a dense masked softmax written
here independently, central finite differences of the oracle's own forward,
SDPA's backward when every block is selected, and the gradient-deficiency
property that motivates SSA (keys outside a query's sparse support get no
gradient from its sparse stream: abstract; Sintesi Tecnica section 1 item 2).
The routing under test: the upstream gradient reaches the active stream only;
L_sparsity moves h_full toward a fixed h_sparse and L_commit moves h_sparse
toward a fixed h_full (Sintesi Tecnica section 2 'Allineamento Bidirezionale').
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY

MODES = [DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY]


def _case(seed, B=1, Hq=4, Hkv=2, N=48, d=6, block=8, K=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    g = rng.standard_normal((B, Hq, N, d))
    sel, _ = oracle.select_blocks(q, k, block, K, Hq // Hkv)
    return q, k, v, g, sel


def _autograd_grads(q, k, v, sel, block, scale, group, mode, dout, w_s, w_c):
    """torch autograd of the SSA layer objective through dense masked softmax."""
    B, Hq, N, d = q.shape
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(group, 1)
    vv = tv.repeat_interleave(group, 1)
    idx = torch.arange(N)
    causal = idx[None, :] <= idx[:, None]
    blk = torch.zeros(B, Hq, N, N // block + 1, dtype=torch.bool)
    s = torch.from_numpy(sel.astype(np.int64))
    s = torch.where(s < 0, torch.full_like(s, N // block), s)
    blk.scatter_(3, s, True)
    sparse = causal & torch.gather(blk, 3, (idx // block).expand(B, Hq, N, N))
    z = scale * tq @ kk.transpose(-1, -2)
    hf = torch.softmax(z.masked_fill(~causal, -math.inf), -1) @ vv
    hs = torch.softmax(z.masked_fill(~sparse, -math.inf), -1) @ vv
    g = torch.from_numpy(dout) if dout is not None else torch.zeros_like(hf)
    if mode == FULL_ONLY:
        J = (g * hf).sum()
    elif mode == SPARSE_ONLY:
        J = (g * hs).sum()
    else:
        active = hf if mode == DUAL_ACTIVE_FULL else hs
        l_sparsity = ((hf - hs.detach()) ** 2).mean()
        l_commit = ((hs - hf.detach()) ** 2).mean()
        J = (g * active).sum() + w_s * l_sparsity + w_c * l_commit
    J.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("mode", MODES)
def test_matches_torch_autograd(mode):
    q, k, v, g, sel = _case(0)
    block, scale, G = 8, 0.45, 2
    ws, wc = 0.7, 1.3
    dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, mode, g, ws, wc)
    rq, rk, rv = _autograd_grads(q, k, v, sel, block, scale, G, mode, g, ws, wc)
    np.testing.assert_allclose(dq, rq, atol=1e-12)
    np.testing.assert_allclose(dk, rk, atol=1e-12)
    np.testing.assert_allclose(dv, rv, atol=1e-12)


@pytest.mark.parametrize("mode", [DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE])
def test_alignment_only_gradients_match_autograd(mode):
    """No upstream gradient: only the alignment terms move q, k, v."""
    q, k, v, _, sel = _case(1)
    block, scale, G = 8, 0.8, 2
    dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, mode, None, 1.0, 1.0)
    rq, rk, rv = _autograd_grads(q, k, v, sel, block, scale, G, mode, None, 1.0, 1.0)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(r).max() > 1e-6
        np.testing.assert_allclose(a, r, atol=1e-15, rtol=1e-9)


def test_finite_differences_of_oracle_forward():
    """<grad, e> equals the central difference of J along random directions e.

    J(q, k, v) = <G_f, h_full> + <G_s, h_sparse> with G_f, G_s fixed at the
    point; the selection stays fixed (it does not depend on v, and the step is
    far below the score margins).
    """
    q, k, v, g, sel = _case(2, Hq=2, Hkv=1, N=32, d=4, block=8, K=2)
    block, scale, G = 8, 0.9, 2
    mode = DUAL_ACTIVE_SPARSE
    f0 = oracle.forward(q, k, v, sel, block, scale, G)
    gf, gs = oracle.stream_grads(mode, g, f0["h_full"], f0["h_sparse"], 1.0, 1.0)
    dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, mode, g, fwd=f0)

    def J(qq, kk, vv):
        f = oracle.forward(qq, kk, vv, sel, block, scale, G)
        return float((gf * f["h_full"]).sum() + (gs * f["h_sparse"]).sum())

    rng = np.random.default_rng(3)
    eps = 1e-6
    for which in range(3):
        for _ in range(3):
            e = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
            e[which] = rng.standard_normal(e[which].shape)
            plus = J(q + eps * e[0], k + eps * e[1], v + eps * e[2])
            minus = J(q - eps * e[0], k - eps * e[1], v - eps * e[2])
            fd = (plus - minus) / (2 * eps)
            an = float((dq * e[0]).sum() + (dk * e[1]).sum() + (dv * e[2]).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_all_blocks_selected_is_sdpa_backward():
    q, k, v, g, _ = _case(4, Hq=4, Hkv=2, N=32, d=8, block=8)
    block, scale, G = 8, 0.35, 2
    sel, _ = oracle.select_blocks(q, k, block, 4, G)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), is_causal=True, scale=scale)
    (out * torch.from_numpy(g)).sum().backward()
    for mode in (FULL_ONLY, SPARSE_ONLY, DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE):
        dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, mode, g)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_gradient_deficiency_of_sparse_stream():
    """One query row's gradient: the sparse stream leaves discarded keys at zero.

    With the upstream gradient on row t only, SPARSE_ONLY gives dk = dv = 0 on
    every causal key outside A_t; the dual modes reach them through the full
    stream (active full) or through L_sparsity on h_full (active sparse).
    """
    q, k, v, _, _ = _case(5, Hq=1, Hkv=1, N=64, d=4, block=8, K=2)
    block, scale = 8, 1.0
    sel, _ = oracle.select_blocks(q, k, block, 2, 1)
    t = 60
    g = np.zeros_like(q)
    g[0, 0, t] = 1.0
    blocks = set(int(x) for x in sel[0, 0, t] if x >= 0)
    outside = [i for i in range(t + 1) if i // block not in blocks]
    assert len(outside) >= 8
    _, dk, dv = oracle.backward(q, k, v, sel, block, scale, 1, SPARSE_ONLY, g)
    assert np.all(dk[0, 0, outside] == 0) and np.all(dv[0, 0, outside] == 0)
    assert np.all(dk[0, 0, t + 1:] == 0) and np.all(dv[0, 0, t + 1:] == 0)
    for mode in (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE):
        _, dk, dv = oracle.backward(q, k, v, sel, block, scale, 1, mode, g)
        assert np.all(np.abs(dv[0, 0, outside]).sum(-1) > 0)
        assert np.all(np.abs(dk[0, 0, outside]).sum(-1) > 0)


def test_gqa_gradients_sum_over_group():
    q, k, v, g, sel = _case(6, Hq=4, Hkv=2, N=32, d=4, block=8, K=2)
    block, scale, G = 8, 0.5, 2
    dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, DUAL_ACTIVE_FULL, g)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    # per-head layer with one KV head each, then fold the group back
    dq1, dk1, dv1 = oracle.backward(q, kr, vr, sel, block, scale, 1, DUAL_ACTIVE_FULL, g)
    np.testing.assert_allclose(dq, dq1, atol=1e-13)
    np.testing.assert_allclose(dk, dk1.reshape(1, 2, G, 32, 4).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv1.reshape(1, 2, G, 32, 4).sum(2), atol=1e-13)


def test_row_sample_helpers_match_full_backward():
    q, k, v, g, sel = _case(7, Hq=4, Hkv=2, N=64, d=4, block=8, K=3)
    block, scale, G = 8, 0.5, 2
    for mode in MODES:
        s = None if mode == FULL_ONLY else sel
        dq, dk, dv = oracle.backward(q, k, v, s, block, scale, G, mode, g, 0.6, 1.7)
        rows = np.array([63, 0, 17])
        dqr = oracle.dq_rows(q, k, v, s, block, scale, G, mode, g, 0, 3, rows, 0.6, 1.7)
        np.testing.assert_allclose(dqr, dq[0, 3, rows], atol=1e-13)
        dkt, dvt = oracle.dkdv_tail(q, k, v, s, block, scale, G, mode, g, 0, 1, 48, 0.6, 1.7)
        np.testing.assert_allclose(dkt, dk[0, 1, 48:], atol=1e-13)
        np.testing.assert_allclose(dvt, dv[0, 1, 48:], atol=1e-13)


def test_sum_properties_any_size():
    """sum_i dk_i = 0 and sum_i dv_i = sum_t (G_f + G_s), per KV head.

    Softmax probabilities sum to one and dZ rows sum to zero; these hold at any
    size and are used for the large-layer GPU checks.
    """
    q, k, v, g, sel = _case(8, Hq=4, Hkv=2, N=64, d=4, block=8, K=3)
    block, scale, G = 8, 0.5, 2
    f = oracle.forward(q, k, v, sel, block, scale, G)
    gf, gs = oracle.stream_grads(DUAL_ACTIVE_SPARSE, g, f["h_full"], f["h_sparse"], 1.0, 1.0)
    dq, dk, dv = oracle.backward(q, k, v, sel, block, scale, G, DUAL_ACTIVE_SPARSE, g, fwd=f)
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-12)
    want = (gf + gs).reshape(1, 2, G, 64, 4).sum((2, 3))
    np.testing.assert_allclose(dv.sum(2), want, atol=1e-12)
