"""The near-tie screening used to make selection parity exact (CPU)."""
import numpy as np

import oracle
import ssa_inputs as si
from oracle.screen import screen_q


def test_screening_removes_near_ties_and_is_deterministic():
    wl = si.WORKLOADS["tiny_mha_n256_fp32"]
    outs = []
    for _ in range(2):
        q, k, v, gen = si.draw_qkv(wl, 0)
        qs, n = screen_q(q, k, wl.block, wl.top_k, wl.group, gen, wl.prescale)
        outs.append((qs, n))
        assert n > 0
        _, margin = oracle.select_blocks(si.to_f64(qs), si.to_f64(k), wl.block, wl.top_k, wl.group)
        assert margin.min() >= 1e-3
        # only failing rows change; the rest keep their original draw
        same = (qs == q).all(-1)
        assert int((~same).sum()) <= n
    assert outs[0][1] == outs[1][1]
    assert bool((outs[0][0] == outs[1][0]).all())


def test_screening_several_cutoffs():
    wl = si.scaled_down(si.WORKLOADS["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=1)
    q, k, v, gen = si.draw_qkv(wl, 3)
    qs, n = screen_q(q, k, wl.block, (2, 4), wl.group, gen, wl.prescale)
    for K in (2, 4):
        _, margin = oracle.select_blocks(si.to_f64(qs), si.to_f64(k), wl.block, K, wl.group)
        assert margin.min() >= 1e-3
