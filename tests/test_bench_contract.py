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


def test_profile_records_are_dropped_when_the_source_changes(tmp_path, monkeypatch):
    """Counter figures (traffic, matrix-pipe use) are reported only while the
    kernel's source is the one they were taken on."""
    import hashlib
    import json

    import bench

    csrc = tmp_path / "block_sparse_full_ssa_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("kernel v1\n")
    sha = hashlib.sha256(b"kernel v1\n").hexdigest()
    rec = {"mfma_util_pct": 50.0, "clock_ghz": 1.5, "executed_bf16_flops": 1.0, "bytes_per_launch": 7,
           "source": "k.hip", "source_sha256": sha}
    for name in ("mfma_util", "hbm_traffic"):
        (tmp_path / "profiles" / f"{name}.json").write_text(json.dumps({"bwd_mfma/w/top_k=16": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.matrix_pipe_use(("bwd_mfma", "bwd_dq"), "w", 16) == {
        "bwd_mfma": {"mfma_util_pct": 50.0, "clock_ghz": 1.5, "executed_bf16_flops": 1.0}, "bwd_dq": None}
    assert bench.measured_traffic("bwd_mfma", "w", 16) == 7
    assert bench.measured_traffic("bwd_mfma", "w", 4) is None
    (csrc / "k.hip").write_text("kernel v2\n")
    assert bench.matrix_pipe_use(("bwd_mfma",), "w", 16) == {"bwd_mfma": None}
    assert bench.measured_traffic("bwd_mfma", "w", 16) is None
