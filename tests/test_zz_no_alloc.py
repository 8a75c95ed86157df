"""ssa_attn_fwd_noalloc (the forward without a workspace argument) against
ssa_attn_fwd, through the C interface.

The no-allocation variant runs the same kernels on a static per-device
workspace, so its outputs must equal those of the workspace entry point bit
for bit.  Two calls in a row, the second on a smaller layer, check that the
shared array carries nothing from one call into the next.
"""
import ctypes
import sys

import pytest
import torch

import ssa_inputs as si

W = si.WORKLOADS
DUAL_FULL, DUAL_SPARSE, FULL_ONLY, SPARSE_ONLY = 0, 1, 2, 3


def _lib():
    from block_sparse_full_ssa_amd import _lib as m
    return m


def _shape(wl, top_k):
    m = _lib()
    return m.ShapeT(wl.batch, wl.hq, wl.group, wl.seqlen, wl.head_dim, wl.block, top_k, 0.0,
                    m.SSA_BF16 if wl.dtype == torch.bfloat16 else m.SSA_F32)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outputs(q, mode):
    B, Hq, N, _ = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    o = {}
    if mode != SPARSE_ONLY:
        o["h_full"] = torch.full_like(q, float("nan"))
        o["lse_full"] = torch.full((B, Hq, N), float("nan"), **f32)
    if mode != FULL_ONLY:
        o["h_sparse"] = torch.full_like(q, float("nan"))
        o["lse_sparse"] = torch.full((B, Hq, N), float("nan"), **f32)
    if mode in (DUAL_FULL, DUAL_SPARSE):
        o["delta"] = torch.full((B, Hq, N), float("nan"), **f32)
        o["losses"] = torch.full((2,), float("nan"), **f32)
    return o


def _call_both(wl, mode, seed=0):
    """(noalloc outputs, workspace-entry outputs) for one layer."""
    L = _lib().lib()
    q, k, v, _ = si.draw_qkv(wl, seed)
    q, k, v = (x.to("cuda:0") for x in (q, k, v))
    sh = _shape(wl, wl.top_k)
    sel = None
    if mode != FULL_ONLY:
        sel = torch.empty(wl.batch, wl.hq, wl.seqlen, wl.top_k, dtype=torch.int32, device="cuda:0")
        n = L.ssa_workspace_size(ctypes.byref(sh), 0, _lib().OP_SELECT)
        ws = torch.empty(n + 256, dtype=torch.uint8, device="cuda:0")
        wp = ws.data_ptr() + (-ws.data_ptr()) % 256
        st = L.ssa_select_blocks(ctypes.byref(sh), _p(q), _p(k), _p(sel), ctypes.c_void_p(wp), n, None)
        assert st == 0, L.ssa_last_error()
    a = _outputs(q, mode)
    st = L.ssa_attn_fwd_noalloc(ctypes.byref(sh), mode, _p(q), _p(k), _p(v), _p(sel), _p(a.get("h_full")),
                                _p(a.get("h_sparse")), _p(a.get("lse_full")), _p(a.get("lse_sparse")),
                                _p(a.get("delta")), _p(a.get("losses")), None)
    assert st == 0, L.ssa_last_error()
    b = _outputs(q, mode)
    n = L.ssa_workspace_size(ctypes.byref(sh), mode, _lib().OP_FWD)
    ws = torch.empty(n + 256, dtype=torch.uint8, device="cuda:0")
    wp = ws.data_ptr() + (-ws.data_ptr()) % 256
    st = L.ssa_attn_fwd(ctypes.byref(sh), mode, _p(q), _p(k), _p(v), _p(sel), _p(b.get("h_full")),
                        _p(b.get("h_sparse")), _p(b.get("lse_full")), _p(b.get("lse_sparse")), _p(b.get("delta")),
                        _p(b.get("losses")), ctypes.c_void_p(wp), n, None)
    assert st == 0, L.ssa_last_error()
    torch.cuda.synchronize()
    return a, b


def _assert_equal(a, b):
    assert a.keys() == b.keys()
    for key in a:
        assert not torch.isnan(a[key]).any(), key
        assert torch.equal(a[key], b[key]), key


@pytest.mark.gpu
def test_noalloc_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [("gqa_n4k dual-sparse", W["gqa_n4k_fwd"], DUAL_SPARSE),
             ("gqa n1024 dual-full", si.scaled_down(W["gqa_n4k_fwd"], seqlen=1024, hq=4, hkv=2, top_k=4), DUAL_FULL),
             ("gqa n512 d64 dual-sparse",
              si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=2, head_dim=64, top_k=4), DUAL_SPARSE)]
    for name, wl, mode in cases:
        print(f"noalloc {name}", flush=True)
        sys.stdout.flush()
        a, b = _call_both(wl, mode)
        _assert_equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [FULL_ONLY, SPARSE_ONLY])
def test_noalloc_single_stream(mode):
    """FULL_ONLY needs no workspace; a small SPARSE_ONLY layer fits the array."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=2, top_k=4)
    print(f"noalloc single stream mode {mode}", flush=True)
    a, b = _call_both(wl, mode)
    _assert_equal(a, b)


@pytest.mark.gpu
def test_noalloc_too_large_rejected_on_gpu():
    """A SPARSE_ONLY layer whose partials exceed the array: SSA_ERR_WORKSPACE,
    nothing enqueued (the outputs keep their contents)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = _lib().lib()
    wl = W["gqa_n4k_fwd"]
    sh = _shape(wl, wl.top_k)
    assert L.ssa_workspace_size(ctypes.byref(sh), SPARSE_ONLY, _lib().OP_FWD) > L.ssa_noalloc_scratch_bytes()
    q, k, v, _ = si.draw_qkv(wl, 0)
    q, k, v = (x.to("cuda:0") for x in (q, k, v))
    sel = torch.zeros(wl.batch, wl.hq, wl.seqlen, wl.top_k, dtype=torch.int32, device="cuda:0")
    o = _outputs(q, SPARSE_ONLY)
    st = L.ssa_attn_fwd_noalloc(ctypes.byref(sh), SPARSE_ONLY, _p(q), _p(k), _p(v), _p(sel), None,
                                _p(o["h_sparse"]), None, _p(o["lse_sparse"]), None, None, None)
    torch.cuda.synchronize()
    assert st == _lib().SSA_ERR_WORKSPACE
    assert b"workspace" in L.ssa_last_error()
    assert torch.isnan(o["h_sparse"]).all()


def test_noalloc_too_large_rejected_on_host():
    """Host-side check, no GPU needed: a dual layer of 16.8M query rows needs
    67 MB of row partials, above the 16 MiB array."""
    import os
    m = _lib()
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libssa not built")
    L = m.lib()
    sh = m.ShapeT(4, 64, 8, 65536, 128, 64, 16, 0.0, m.SSA_BF16)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the call fails before any launch
    st = L.ssa_attn_fwd_noalloc(ctypes.byref(sh), DUAL_FULL, fake, fake, fake, fake, fake, fake, fake, fake,
                                fake, fake, None)
    assert st == m.SSA_ERR_WORKSPACE
    assert L.ssa_noalloc_scratch_bytes() == 16 << 20
