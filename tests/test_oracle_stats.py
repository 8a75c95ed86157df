"""Pins of the oracle's full-stream diagnostics: the sink-block mass and the
entropy of the full attention distribution (CPU).

Independent references: closed forms for q = 0 (uniform attention), scipy's
entropy of torch's float64 softmax, a planted dominant key (all mass on the
sink block, entropy near zero), and the invariants 0 <= H <= ln(t+1),
0 <= sink <= 1 with sink = 1 for every row inside the first block.
"""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle


def test_zero_queries_closed_form():
    """q = 0: p_f(t, .) is uniform over t + 1 keys."""
    rng = np.random.default_rng(3)
    B, Hq, N, d, block = 1, 2, 50, 4, 8
    q = np.zeros((B, Hq, N, d))
    k = rng.standard_normal((B, 1, N, d))
    sink, ent, means = oracle.full_stats(q, k, block, 0.5, 2)
    for t in range(N):
        assert abs(ent[0, 0, t] - math.log(t + 1)) < 1e-13
        assert abs(sink[0, 1, t] - min(block, t + 1) / (t + 1)) < 1e-14
    np.testing.assert_allclose(means[0, :, 1], np.mean([math.log(t + 1) for t in range(N)]), atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_against_torch_softmax_and_scipy_entropy(seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d, block, scale = 2, 4, 2, 70, 16, 16, 0.7
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    sink, ent, means = oracle.full_stats(q, k, block, scale, Hq // Hkv)
    for b in range(B):
        for h in range(Hq):
            kc = torch.from_numpy(k[b, h // (Hq // Hkv)])
            z = scale * (torch.from_numpy(q[b, h]) @ kc.T)
            z = z.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
            p = torch.softmax(z, dim=1).numpy()
            for t in range(N):
                assert abs(ent[b, h, t] - scipy.stats.entropy(p[t, :t + 1])) < 1e-12
                assert abs(sink[b, h, t] - p[t, :block].sum()) < 1e-13
    np.testing.assert_allclose(means[..., 0], sink.mean(axis=2), atol=1e-15)
    np.testing.assert_allclose(means[..., 1], ent.mean(axis=2), atol=1e-15)


def test_planted_dominant_sink_key():
    """Key 0 aligned with every query at logit ~60 above the rest: all mass on
    the first block, entropy ~0 (rows t >= 1)."""
    rng = np.random.default_rng(5)
    B, N, d, block = 1, 64, 8, 16
    u = np.zeros(d)
    u[0] = 1.0
    q = np.tile(u, (B, 1, N, 1)) + 0.01 * rng.standard_normal((B, 1, N, d))
    k = 0.01 * rng.standard_normal((B, 1, N, d))
    k[0, 0, 0] = 60.0 * u
    sink, ent, _ = oracle.full_stats(q, k, block, 1.0, 1)
    assert np.all(np.abs(sink[0, 0] - 1.0) < 1e-12)
    assert np.all(ent[0, 0, 1:] < 1e-20)


def test_invariants_random():
    rng = np.random.default_rng(9)
    B, Hq, N, d, block = 1, 3, 100, 8, 32
    q = 2.0 * rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hq, N, d))
    sink, ent, _ = oracle.full_stats(q, k, block, 1.0, 1)
    t = np.arange(N)
    assert np.all(ent >= -1e-15) and np.all(ent <= np.log(t + 1) + 1e-12)
    assert np.all(sink >= 0) and np.all(sink <= 1 + 1e-15)
    assert np.all(np.abs(sink[..., :block] - 1.0) < 1e-15)
