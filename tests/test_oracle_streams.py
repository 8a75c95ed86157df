"""Pins of the oracle's two attention streams, delta(t) and the losses (CPU).

Independent references: torch's scaled_dot_product_attention in float64, a
brute-force N x N masked softmax built from an exhaustive selection, closed
forms for q = 0, and the decomposition of the full output into the selected
and the discarded parts (the error of sparse attention is linear in the
discarded mass: Sintesi Tecnica, section 1 and section 3 'Framework
Teorico').
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import DUAL_ACTIVE_FULL, FULL_ONLY, SPARSE_ONLY


def _rand(seed, B=1, Hq=4, Hkv=2, N=64, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    return q, k, v


def _sdpa(q, k, v, scale, mask=None, causal=False, group=1):
    """torch SDPA in float64; GQA by repeating each KV head ``group`` times."""
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(group, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(group, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, is_causal=causal, scale=scale)
    return out.numpy()


@pytest.mark.parametrize("seed", [0, 1])
def test_all_blocks_selected_equals_full_equals_sdpa(seed):
    q, k, v = _rand(seed)
    block, G, scale = 8, 2, 0.4
    nb = q.shape[2] // block
    for K in (nb, nb + 3):
        sel, _ = oracle.select_blocks(q, k, block, K, G)
        f = oracle.forward(q, k, v, sel, block, scale, G)
        ref = _sdpa(q, k, v, scale, causal=True, group=G)
        np.testing.assert_allclose(f["h_full"], ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(f["h_sparse"], ref, atol=1e-12, rtol=0)
        assert np.all(f["delta"] == 0.0)
        assert f["L_sparsity"] == 0.0 and f["L_commit"] == 0.0
        np.testing.assert_array_equal(f["lse_full"], f["lse_sparse"])


def _brute_force_sel(q, k, block, K, group):
    """Exhaustive subset search per row (tiny sizes only)."""
    B, Hq, N, d = q.shape
    nb = N // block
    sel = np.full((B, Hq, N, K), -1, np.int32)
    for b in range(B):
        for h in range(Hq):
            mu = k[b, h // group].reshape(nb, block, d).mean(axis=1)
            for t in range(N):
                i = t // block
                sig = mu @ q[b, h, t]
                best, bs = None, -np.inf
                for comb in itertools.combinations(range(i), min(K - 1, i)):
                    s = float(sum(sig[j] for j in comb))
                    if s > bs:
                        best, bs = comb, s
                row = sorted(set(best) | {i})
                sel[b, h, t, :len(row)] = row
    return sel


def _dense_masks(sel, N, block):
    """Causal and sparse-support masks [B, H, N, N] built key by key."""
    B, H = sel.shape[:2]
    causal = np.zeros((N, N), bool)
    sparse = np.zeros((B, H, N, N), bool)
    for t in range(N):
        for i in range(t + 1):
            causal[t, i] = True
    for b in range(B):
        for h in range(H):
            for t in range(N):
                blocks = set(int(x) for x in sel[b, h, t] if x >= 0)
                for i in range(t + 1):
                    if i // block in blocks:
                        sparse[b, h, t, i] = True
    return causal, sparse


@pytest.mark.parametrize("K", [1, 2, 3])
def test_brute_force_masked_softmax(K):
    q, k, v = _rand(3, Hq=4, Hkv=2, N=24, d=5)
    block, G, scale = 4, 2, 0.7
    sel = _brute_force_sel(q, k, block, K, G)
    osel, _ = oracle.select_blocks(q, k, block, K, G)
    np.testing.assert_array_equal(osel, sel)
    f = oracle.forward(q, k, v, sel, block, scale, G)
    N = q.shape[2]
    causal, sparse = _dense_masks(sel, N, block)
    kk = torch.from_numpy(k).repeat_interleave(G, 1)
    vv = torch.from_numpy(v).repeat_interleave(G, 1)
    z = scale * torch.from_numpy(q) @ kk.transpose(-1, -2)
    zf = z.masked_fill(~torch.from_numpy(causal), -math.inf)
    zs = z.masked_fill(~torch.from_numpy(sparse), -math.inf)
    pf, ps = torch.softmax(zf, -1), torch.softmax(zs, -1)
    np.testing.assert_allclose(f["h_full"], (pf @ vv).numpy(), atol=1e-12)
    np.testing.assert_allclose(f["h_sparse"], (ps @ vv).numpy(), atol=1e-12)
    np.testing.assert_allclose(f["lse_full"], torch.logsumexp(zf, -1).numpy(), atol=1e-12)
    np.testing.assert_allclose(f["lse_sparse"], torch.logsumexp(zs, -1).numpy(), atol=1e-12)
    disc = torch.from_numpy(causal & ~sparse)
    np.testing.assert_allclose(f["delta"], (pf * disc).sum(-1).numpy(), atol=1e-12)
    L = float(((pf @ vv - ps @ vv) ** 2).mean())
    assert abs(f["L_sparsity"] - L) <= 1e-12 * max(1.0, L)


def test_top1_is_block_diagonal_attention():
    """K = 1 keeps only the own block: block-diagonal causal attention."""
    q, k, v = _rand(4, Hq=2, Hkv=1, N=32, d=6)
    block, scale = 8, 0.5
    sel, _ = oracle.select_blocks(q, k, block, 1, 2)
    f = oracle.forward(q, k, v, sel, block, scale, 2)
    t = np.arange(32)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] // block == t[:, None] // block)
    ref = _sdpa(q, k, v, scale, mask=mask, group=2)
    np.testing.assert_allclose(f["h_sparse"], ref, atol=1e-12)


def test_zero_queries_closed_form():
    """q = 0: uniform weights, so outputs are plain means and delta is a count.

    h_full[t] = mean of v[0..t]; h_sparse[t] = mean of v over A_t;
    delta(t) = 1 - |A_t| / (t + 1).
    """
    rng = np.random.default_rng(6)
    B, Hq, N, d, block, K = 1, 1, 40, 3, 5, 3
    q = np.zeros((B, Hq, N, d))
    k = rng.standard_normal((B, 1, N, d))
    v = rng.standard_normal((B, 1, N, d))
    sel, _ = oracle.select_blocks(q, k, block, K, 1)
    f = oracle.forward(q, k, v, sel, block, 1.0, 1)
    for t in range(N):
        i = t // block
        keep = set(range(min(K - 1, i))) | {i}           # ties -> lowest blocks
        A = [j for j in range(t + 1) if j // block in keep]
        np.testing.assert_allclose(f["h_full"][0, 0, t], v[0, 0, :t + 1].mean(0), atol=1e-14)
        np.testing.assert_allclose(f["h_sparse"][0, 0, t], v[0, 0, A].mean(0), atol=1e-14)
        assert abs(f["delta"][0, 0, t] - (1 - len(A) / (t + 1))) < 1e-14
        assert abs(f["lse_full"][0, 0, t] - math.log(t + 1)) < 1e-13
        assert abs(f["lse_sparse"][0, 0, t] - math.log(len(A))) < 1e-13


def test_hand_worked_two_blocks():
    """N = 4, block = 2, top_k = 1, d = 1: every number written out by hand.

    q = [1, 2, 3, 4] / 4, k = [1, -1, 2, 0], v = [10, 20, 30, 40], scale = 1.
    Row t = 3: full logits z = q3 * k = [1, -1, 2, 0] over keys 0..3; the
    sparse support is the own block {2, 3} with logits [2, 0].
    """
    q = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 4, 1) / 4
    k = np.array([1.0, -1.0, 2.0, 0.0]).reshape(1, 1, 4, 1)
    v = np.array([10.0, 20.0, 30.0, 40.0]).reshape(1, 1, 4, 1)
    sel, _ = oracle.select_blocks(q, k, 2, 1, 1)
    f = oracle.forward(q, k, v, sel, 2, 1.0, 1)
    e = math.exp
    zf = [e(1), e(-1), e(2), e(0)]
    hf3 = (10 * zf[0] + 20 * zf[1] + 30 * zf[2] + 40 * zf[3]) / sum(zf)
    hs3 = (30 * e(2) + 40 * e(0)) / (e(2) + e(0))
    d3 = (zf[0] + zf[1]) / sum(zf)
    assert abs(f["h_full"][0, 0, 3, 0] - hf3) < 1e-12
    assert abs(f["h_sparse"][0, 0, 3, 0] - hs3) < 1e-12
    assert abs(f["delta"][0, 0, 3] - d3) < 1e-15
    assert abs(f["lse_full"][0, 0, 3] - math.log(sum(zf))) < 1e-14
    # row 2 (first key of block 1): sparse sees key 2 only -> v2 exactly
    assert f["h_sparse"][0, 0, 2, 0] == 30.0
    zf2 = [e(0.75), e(-0.75), e(1.5)]
    assert abs(f["delta"][0, 0, 2] - (zf2[0] + zf2[1]) / sum(zf2)) < 1e-15
    # rows 0, 1 see only block 0, which is their own block -> no discarded mass
    assert f["delta"][0, 0, 0] == 0.0 and f["delta"][0, 0, 1] == 0.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_delta_decomposition_and_bound(seed):
    """h_full - h_sparse = delta (h_u - h_sparse), and |.| <= 2 delta max|v|.

    h_u is attention restricted to the discarded keys, computed separately
    with SDPA and an explicit complement mask.  Also delta = 1 - exp(lse_s -
    lse_f) and p_sparse = p_full / (1 - delta) on the selected keys.
    """
    q, k, v = _rand(seed, Hq=2, Hkv=1, N=96, d=8)
    q *= 2.0
    block, G, K, scale = 8, 2, 3, 0.6
    sel, _ = oracle.select_blocks(q, k, block, K, G)
    f = oracle.forward(q, k, v, sel, block, scale, G)
    N = q.shape[2]
    causal, sparse = _dense_masks(sel, N, block)
    comp = causal[None, None] & ~sparse
    has = comp.any(-1)                                   # rows with discarded keys
    safe = np.where(has[..., None], comp, np.eye(N, dtype=bool)[None, None])
    hu = _sdpa(q, k, v, scale, mask=safe, group=G)
    delta = f["delta"]
    lhs = f["h_full"] - f["h_sparse"]
    rhs = delta[..., None] * (hu - f["h_sparse"])
    rhs = np.where(has[..., None], rhs, 0.0)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    vmax = np.linalg.norm(v, axis=-1).max()
    assert np.all(np.linalg.norm(lhs, axis=-1) <= 2 * delta * vmax + 1e-12)
    np.testing.assert_allclose(delta, -np.expm1(f["lse_sparse"] - f["lse_full"]), atol=1e-13)
    assert np.all(delta >= 0) and np.all(delta < 1)
    t = np.arange(N)
    assert np.all(delta[:, :, t // block < K] == 0.0)
    assert np.any(delta[:, :, t // block >= K] > 1e-3)


def test_single_stream_modes_match_dual():
    q, k, v = _rand(8, Hq=4, Hkv=2, N=48, d=8)
    block, G, K, scale = 8, 2, 2, 0.3
    sel, _ = oracle.select_blocks(q, k, block, K, G)
    d = oracle.forward(q, k, v, sel, block, scale, G, DUAL_ACTIVE_FULL)
    fo = oracle.forward(q, k, v, None, block, scale, G, FULL_ONLY)
    so = oracle.forward(q, k, v, sel, block, scale, G, SPARSE_ONLY)
    assert set(fo) == {"h_full", "lse_full"} and set(so) == {"h_sparse", "lse_sparse"}
    np.testing.assert_array_equal(fo["h_full"], d["h_full"])
    np.testing.assert_array_equal(so["h_sparse"], d["h_sparse"])


def test_losses_equal_and_closed_form():
    """Both losses equal the mean of (h_full - h_sparse)^2; q = 0 closed form."""
    rng = np.random.default_rng(11)
    N, d, block, K = 30, 2, 5, 2
    q = np.zeros((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    sel, _ = oracle.select_blocks(q, k, block, K, 1)
    f = oracle.forward(q, k, v, sel, block, 1.0, 1)
    tot = 0.0
    for t in range(N):
        i = t // block
        keep = {0, i} if i >= 1 else {0}
        A = [j for j in range(t + 1) if j // block in keep]
        diff = v[0, 0, :t + 1].mean(0) - v[0, 0, A].mean(0)
        tot += float(diff @ diff)
    assert f["L_sparsity"] == f["L_commit"]
    assert abs(f["L_sparsity"] - tot / (N * d)) < 1e-14


def test_attend_rows_sample_matches_full_forward():
    q, k, v = _rand(12, Hq=2, Hkv=1, N=80, d=4)
    block, G, K, scale = 8, 2, 3, 0.5
    sel, _ = oracle.select_blocks(q, k, block, K, G)
    f = oracle.forward(q, k, v, sel, block, scale, G)
    rows = np.array([79, 5, 33])
    o = oracle.attend_rows(q[0, 1, rows], rows, k[0, 0], v[0, 0], sel[0, 1, rows], block, scale)
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta"):
        np.testing.assert_allclose(o[key], f[key][0, 1, rows], atol=1e-13)
