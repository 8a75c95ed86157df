"""Pins of the oracle's block selection (CPU only).

Selection rule (fixed where the pages leave it open): block j < i_t of query t
scores q_t . mean(k over block j); the own block i_t is always kept; the other
top_k - 1 slots go to the highest scores, a lower block index winning a tie.
"""
import itertools

import numpy as np
import pytest

from oracle import block_means, select_blocks, select_rows


def _keys_with_block_means(means, block, rng):
    """Keys whose per-block means are exactly ``means`` [nb, d].

    Each block gets zero-mean noise (pairs of +e, -e) added to its mean, so the
    block means are exact in floating point only up to rounding; the noise is
    drawn from small dyadic values so every sum is exact.
    """
    nb, d = means.shape
    k = np.repeat(means, block, axis=0).copy()
    noise = rng.integers(-4, 5, size=(nb, block // 2, d)) / 8.0
    k[:, :] += 0.0
    k = k.reshape(nb, block, d)
    k[:, 0::2, :] += noise
    k[:, 1::2, :] -= noise
    return k.reshape(nb * block, d)


def test_block_means_plain():
    k = np.arange(2 * 8 * 3, dtype=np.float64).reshape(1, 2, 8, 3)
    mu = block_means(k, 4)
    assert mu.shape == (1, 2, 2, 3)
    # block 0 of head 0 holds rows 0..3 = values 0..11 -> mean of rows is row 1.5
    np.testing.assert_array_equal(mu[0, 0, 0], [4.5, 5.5, 6.5])
    np.testing.assert_array_equal(mu[0, 1, 1], k[0, 1, 4:8].mean(axis=0))


def test_planted_ranking_hand_worked():
    """Block means c_j * u with q = u: ranking is the order of c, known by hand.

    nb = 6, block = 4, d = 3, top_k = 3 (own block + 2), c = [3, 0, 5, 1, 4, 2].
      block 0 rows: candidates none            -> [0]
      block 1 rows: candidates {0}             -> [0, 1]
      block 2 rows: candidates {0, 1}          -> [0, 1, 2]
      block 3 rows: c(0..2) = 3, 0, 5 -> 2, 0  -> [0, 2, 3]
      block 4 rows: c(0..3) = 3, 0, 5, 1 -> 2, 0 -> [0, 2, 4]
      block 5 rows: c(0..4) = 3, 0, 5, 1, 4 -> 2, 4 -> [2, 4, 5]
    """
    rng = np.random.default_rng(1)
    block, d = 4, 3
    u = np.array([0.5, -1.0, 0.25])
    c = np.array([3.0, 0.0, 5.0, 1.0, 4.0, 2.0])
    k = _keys_with_block_means(c[:, None] * u[None, :], block, rng)
    N = k.shape[0]
    q = np.tile(u, (N, 1))
    sel, margin = select_blocks(q[None, None], k[None, None], block, 3, 1)
    expect = {0: [0, -1, -1], 1: [0, 1, -1], 2: [0, 1, 2], 3: [0, 2, 3], 4: [0, 2, 4], 5: [2, 4, 5]}
    for t in range(N):
        assert list(sel[0, 0, t]) == expect[t // block], t
    # margins: |u|^2 = 1.3125 times the score gap at the cutoff
    uu = float(u @ u)
    assert np.all(np.isinf(margin[0, 0, :12]))
    np.testing.assert_allclose(margin[0, 0, 12:16], (3 - 0) * uu)   # kept c=3, dropped c=0
    np.testing.assert_allclose(margin[0, 0, 16:20], (3 - 1) * uu)   # kept c=3, dropped c=1
    np.testing.assert_allclose(margin[0, 0, 20:24], (4 - 3) * uu)   # kept c=4, dropped c=3


def test_ties_lower_index_wins():
    """q = 0 makes every score 0: the lowest K-1 earlier blocks are kept."""
    rng = np.random.default_rng(2)
    B, H, N, d, block, K = 1, 2, 64, 8, 8, 4
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    sel, margin = select_blocks(q, k, block, K, 1)
    for t in range(N):
        i = t // block
        want = sorted(set(range(min(K - 1, i))) | {i})
        row = list(sel[0, 1, t])
        assert row[:len(want)] == want and all(x == -1 for x in row[len(want):])
    assert np.all(margin[:, :, 4 * block:] == 0.0)


def _brute_force_row(sigma, i, K):
    """Max-sum (K-1)-subset of candidates 0..i-1, lexicographically smallest on ties."""
    keep = min(K - 1, i)
    best, best_sum = None, -np.inf
    for comb in itertools.combinations(range(i), keep):   # lexicographic order
        s = float(sum(sigma[j] for j in comb))
        if s > best_sum:
            best, best_sum = comb, s
    return sorted(set(best) | {i})


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_brute_force_subsets(seed, K):
    """Enumerate every subset on a tiny layer; integer-valued scores force ties."""
    rng = np.random.default_rng(seed)
    block, nb, d = 2, 7, 3
    N = block * nb
    q = rng.integers(-2, 3, size=(1, 2, N, d)).astype(np.float64)
    k = rng.integers(-2, 3, size=(1, 1, N, d)).astype(np.float64) * 2.0
    sel, _ = select_blocks(q, k, block, K, 2)
    mu = k[0, 0].reshape(nb, block, d).mean(axis=1)
    for h in range(2):
        for t in range(N):
            i = t // block
            sigma = mu @ q[0, h, t]
            want = _brute_force_row(sigma, i, K)
            got = [x for x in sel[0, h, t] if x >= 0]
            assert got == want, (h, t, sigma[:i], got, want)


def test_matches_numpy_lexsort():
    """Library cross-check: rank by numpy.lexsort((j, -sigma))."""
    rng = np.random.default_rng(5)
    block, nb, d, K = 4, 16, 8, 6
    N = block * nb
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    sel, _ = select_blocks(q, k, block, K, 1)
    mu = k[0, 0].reshape(nb, block, d).mean(axis=1)
    for t in range(N):
        i = t // block
        sig = mu[:i] @ q[0, 0, t]
        j = np.arange(i)
        order = np.lexsort((j, -sig))[:K - 1]
        want = sorted(set(order.tolist()) | {i})
        assert [x for x in sel[0, 0, t] if x >= 0] == want


def test_gqa_uses_group_kv_head():
    rng = np.random.default_rng(7)
    block, nb, d, K, G = 4, 8, 4, 3, 2
    N = block * nb
    q = rng.standard_normal((1, 4, N, d))
    k = rng.standard_normal((1, 2, N, d))
    sel, _ = select_blocks(q, k, block, K, G)
    for h in range(4):
        s1, _ = select_blocks(q[:, h:h + 1], k[:, h // G:h // G + 1], block, K, 1)
        np.testing.assert_array_equal(sel[:, h], s1[:, 0])


def test_topk_larger_than_blocks_selects_all():
    rng = np.random.default_rng(8)
    block, nb, d = 4, 5, 4
    N = block * nb
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    sel, margin = select_blocks(q, k, block, 9, 1)
    for t in range(N):
        i = t // block
        assert list(sel[0, 0, t, :i + 1]) == list(range(i + 1))
        assert np.all(sel[0, 0, t, i + 1:] == -1)
    assert np.all(np.isinf(margin))


def test_select_rows_subset_matches_all_rows():
    rng = np.random.default_rng(9)
    block, nb, d, K = 8, 9, 5, 4
    N = block * nb
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((1, 1, N, d))
    mu = block_means(k, block)[0, 0]
    all_sel, all_m = select_rows(q, np.arange(N), mu, block, K)
    rows = np.array([70, 3, 40, 41, 9])
    s, m = select_rows(q[rows], rows, mu, block, K)
    np.testing.assert_array_equal(s, all_sel[rows])
    np.testing.assert_array_equal(m, all_m[rows])
