"""Host-side checks of the benchmark's contract (no GPU needed).

bench.py measures one GPU: asked for more it must exit with a message before
touching any device, and the algorithmic counts it divides by must follow
the per-pair convention (4d forward + 10d backward flops per causal pair,
both streams) with the pair counts of the causal and block-sparse supports.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("N, block, K", [(16384, 64, 4), (16384, 64, 16), (16384, 64, 32), (65536, 64, 32),
                                         (256, 32, 4)])
def test_pair_counts_match_brute_force_on_block_grid(N, block, K):
    """P_full = N (N + 1) / 2 and P_sparse = sum over queries of the keys in
    their selected blocks (own block up to the query, plus min(K - 1, i)
    whole earlier blocks), counted directly per query block."""
    import bench

    pf, ps = bench.pairs(N, block, K)
    assert pf == N * (N + 1) // 2
    nb = N // block
    want = 0
    for i in range(nb):
        earlier = min(K - 1, i) * block          # whole earlier blocks per query
        own = block * (block + 1) // 2           # the own block, causal, summed over its queries
        want += block * earlier + own
    assert ps == want


def test_headline_flops_per_step():
    """The 16K layer at top_k 16: 14 d (P_full + P_sparse) B Hq = 1.720e13."""
    import bench

    pf, ps = bench.pairs(16384, 64, 16)
    assert (pf, ps) == (134225920, 15769600)
    assert abs(14 * 128 * (pf + ps) * 2 * 32 - 1.7203e13) < 1e10
