"""Shared helpers of the GPU parity tests: screened inputs, oracle results
(cached per case), and the tolerance checks.

Tolerances (element-wise |x - ref| <= atol + rtol |ref|): bf16 layers atol
2e-2, rtol 1e-2; the fp32 layer 1e-5 / 1e-5.  Scalars (the losses) use the
relative part only.  Gradients that come from the alignment losses alone are
about 1/M in size, so those checks are normwise:
max |x - ref| <= rtol * max |ref|.
"""
from __future__ import annotations

import functools
import math

import numpy as np
import torch

import oracle
import ssa_inputs as si
from oracle.screen import screen_q

TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-5, 1e-5)}


def scale_of(wl) -> float:
    return 1.0 / math.sqrt(wl.head_dim)


@functools.lru_cache(maxsize=None)
def inputs(wl, seed: int, screen_ks: tuple):
    """Screened q, k, v (CPU tensors) and their exact float64 copies."""
    q, k, v, gen = si.draw_qkv(wl, seed)
    if screen_ks:
        q, _ = screen_q(q, k, wl.block, screen_ks, wl.group, gen, wl.prescale)
    return (q, k, v), tuple(si.to_f64(x) for x in (q, k, v))


@functools.lru_cache(maxsize=None)
def oracle_select(wl, seed, screen_ks, top_k):
    _, (qf, kf, vf) = inputs(wl, seed, screen_ks)
    sel, margin = oracle.select_blocks(qf, kf, wl.block, top_k, wl.group)
    return sel, margin


@functools.lru_cache(maxsize=None)
def oracle_fwd(wl, seed, screen_ks, top_k, mode):
    _, (qf, kf, vf) = inputs(wl, seed, screen_ks)
    sel = oracle_select(wl, seed, screen_ks, top_k)[0] if mode != oracle.FULL_ONLY else None
    return oracle.forward(qf, kf, vf, sel, wl.block, scale_of(wl), wl.group, mode)


def to_dev(*xs):
    return [x.to("cuda:0") for x in xs]


def excess(got, want, atol, rtol):
    """Largest amount by which |got - want| exceeds atol + rtol |want| (<= 0 passes)."""
    g = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    return float((np.abs(g - want) - (atol + rtol * np.abs(want))).max())


def assert_close(name, got, want, dtype):
    atol, rtol = TOL[dtype]
    g = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    ex = np.abs(g - want) - (atol + rtol * np.abs(want))
    e = float(ex.max()) if ex.size else 0.0
    if e > 0:
        at = np.unravel_index(int(np.argmax(ex)), ex.shape)
        bad = int((ex > 0).sum())
        raise AssertionError(f"{name}: exceeds tolerance by {e:.3g} at {tuple(int(i) for i in at)} "
                             f"(got {g[at]:.6g}, want {want[at]:.6g}; {bad} elements out of tolerance)")


def assert_normwise(name, got, want, rtol):
    g = got.detach().float().cpu().numpy()
    err = np.abs(g - want).max()
    ref = np.abs(want).max()
    assert ref > 0 and err <= rtol * ref, f"{name}: normwise error {err / max(ref, 1e-300):.3g}"


MARGIN = 1e-3


def check_selection(name, q_rows, t_idx, mu_c, block, K, gpu_rows):
    """Equal to the oracle where the fp64 margin is >= MARGIN; elsewhere a
    valid selection whose scores are within MARGIN of the optimum."""
    ref, margin = oracle.select_rows(q_rows, t_idx, mu_c, block, K)
    ok = margin >= MARGIN
    bad = np.nonzero(ok & np.any(ref != gpu_rows, axis=1))[0]
    assert bad.size == 0, f"{name}: selection differs on rows {t_idx[bad][:8]}"
    for r in np.nonzero(~ok)[0]:
        t, i = int(t_idx[r]), int(t_idx[r]) // block
        row = gpu_rows[r]
        kept = row[row >= 0]
        assert kept.size == min(K, i + 1) and np.all(np.diff(kept) > 0) and kept[-1] == i, (name, t, row)
        sigma = q_rows[r] @ mu_c[:i].T
        cutoff = np.sort(sigma)[::-1][min(K - 1, i) - 1]
        assert np.all(sigma[kept[:-1]] >= cutoff - MARGIN), (name, t)
    return int((~ok).sum())
