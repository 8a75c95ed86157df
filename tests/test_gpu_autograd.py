"""The torch.autograd binding (SSAFunction / ssa_attention) against the oracle.

The objective <dO, h_active> + w_s L_sparsity + w_c L_commit is
differentiated by torch autograd through the library's forward and backward;
the gradients of q, k and v must equal the oracle's explicit backward with
the upstream gradient on the active output only and the stop-gradient routing
of the two alignment losses (Sintesi Tecnica, section 2, 'Allineamento
Bidirezionale', items 1 and 2).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import ssa_inputs as si

from gpu_cases import assert_close, assert_normwise, inputs, oracle_fwd, oracle_select, scale_of, to_dev

pytestmark = pytest.mark.gpu

W = si.WORKLOADS
TINY = W["tiny_mha_n256_fp32"]
SMALL_BF16 = si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=2, top_k=4)
SMALL_BF16_D64 = si.scaled_down(W["gqa_n4k_fwd"], seqlen=384, hq=4, hkv=2, head_dim=64, block=32, top_k=3)
ACTIVE = {oracle.DUAL_ACTIVE_FULL: "h_full", oracle.DUAL_ACTIVE_SPARSE: "h_sparse",
          oracle.FULL_ONLY: "h_full", oracle.SPARSE_ONLY: "h_sparse"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_full_ssa_amd  # noqa: F401


def _run(wl, mode, ws, wc, with_dout=True):
    import block_sparse_full_ssa_amd as ssa

    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    g = si.draw_dout(wl, 0)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    for t in (qd, kd, vd):
        t.requires_grad_(True)
    out = ssa.ssa_attention(qd, kd, vd, wl.block, wl.top_k, mode)
    obj = ws * out.losses[0] + wc * out.losses[1]
    if with_dout:
        obj = obj + (gd.float() * out.h.float()).sum()
    obj.backward()
    torch.cuda.synchronize()
    osel = oracle_select(wl, 0, (wl.top_k,), wl.top_k)[0]
    if mode != oracle.FULL_ONLY:
        assert np.array_equal(out.sel.cpu().numpy(), osel)
    ref = oracle_fwd(wl, 0, (wl.top_k,), wl.top_k, mode)
    dual = mode in (oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE)
    rq, rk, rv = oracle.backward(qf, kf, vf, None if mode == oracle.FULL_ONLY else osel, wl.block,
                                 scale_of(wl), wl.group, mode, si.to_f64(g) if with_dout else None,
                                 ws if dual else 0.0, wc if dual else 0.0, fwd=ref)
    return out, ref, (qd.grad, kd.grad, vd.grad), (rq, rk, rv)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE, oracle.FULL_ONLY,
                                  oracle.SPARSE_ONLY])
@pytest.mark.parametrize("name", ["tiny", "bf16", "bf16_d64"])
def test_autograd_matches_oracle(name, mode):
    wl = {"tiny": TINY, "bf16": SMALL_BF16, "bf16_d64": SMALL_BF16_D64}[name]
    print(f"autograd {name} mode {mode}", flush=True)
    sys.stdout.flush()
    out, ref, got, want = _run(wl, mode, 0.7, 1.3)
    assert_close("h", out.h, ref[ACTIVE[mode]], wl.dtype)
    if mode in (oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE):
        L = out.losses.detach().cpu().numpy()
        assert L[0] == L[1]
        assert abs(L[0] - ref["L_sparsity"]) <= 1e-2 * ref["L_sparsity"]
        assert_close("delta", out.delta, ref["delta"], wl.dtype)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_close(f"{name} {n}", a, b, wl.dtype)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE])
def test_autograd_alignment_only(mode):
    """Only the two losses in the objective: their gradients reach q, k, v
    through both streams, each loss through the output it moves."""
    out, ref, got, want = _run(TINY, mode, 1.0, 0.5, with_dout=False)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_normwise(f"align {n}", a, b, 1e-4)


def test_autograd_losses_only_sparsity():
    """L_sparsity alone moves only h_full: with no upstream gradient and
    w_commit = 0 the sparse stream receives nothing."""
    out, ref, got, want = _run(TINY, oracle.DUAL_ACTIVE_SPARSE, 1.0, 0.0, with_dout=False)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_normwise(f"sparsity-only {n}", a, b, 1e-4)
