"""The C interface of libssa on the host: symbols, workspace sizes, and the
argument validation that runs before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from block_sparse_full_ssa_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_full_ssa_amd import build
        build.build(verbose=False)
    return _lib.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ssa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert "ssa_attn_fwd" in names and "ssa_attn_bwd" in names and "ssa_select_blocks" in names
    for n in names:
        assert hasattr(L, n), n
    from block_sparse_full_ssa_amd import _lib
    assert sorted(_lib.EXPORTED) == names


def _shape(**kw):
    from block_sparse_full_ssa_amd import _lib
    d = dict(batch=1, heads_q=4, group=2, seqlen=256, head_dim=128, block=64, top_k=4,
             softmax_scale=0.0, dtype=_lib.SSA_BF16)
    d.update(kw)
    return _lib.ShapeT(**d)


def test_workspace_sizes(L):
    from block_sparse_full_ssa_amd import _lib
    s = _shape()
    sel_ws = L.ssa_workspace_size(ctypes.byref(s), 0, _lib.OP_SELECT)
    assert sel_ws >= 2 * 128 * 4 * 4          # B*Hkv*d*nb fp32 block means
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, _lib.OP_FWD) >= 4 * 256 * 4
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.FULL_ONLY, _lib.OP_FWD) == 0
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, _lib.OP_BWD) > 0
    bad = _shape(seqlen=100)
    assert L.ssa_workspace_size(ctypes.byref(bad), 0, _lib.OP_FWD) == 0
    assert L.ssa_workspace_size(ctypes.byref(s), 7, _lib.OP_FWD) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,status", [
    (dict(seqlen=100), 2),             # N % block
    (dict(group=3), 2),                # group does not divide heads_q
    (dict(top_k=0), 2),
    (dict(batch=0), 2),
    (dict(head_dim=96), 3),
    (dict(block=48), 3),
    (dict(dtype=5), 3),
    (dict(top_k=65, seqlen=64 * 100), 3),
    (dict(seqlen=64 * 4097), 3),       # more than 4096 key blocks
])
def test_shape_errors(L, kw, status):
    s = _shape(**kw)
    st = L.ssa_select_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status, L.ssa_last_error()
    assert L.ssa_last_error().decode()
    st = L.ssa_attn_fwd(ctypes.byref(s), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, 1 << 30, None)
    assert st == status


def test_null_and_workspace_errors(L):
    from block_sparse_full_ssa_amd import _lib
    s = _shape()
    assert L.ssa_select_blocks(None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.SSA_ERR_NULL
    assert L.ssa_select_blocks(ctypes.byref(s), None, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.SSA_ERR_NULL
    # workspace: too small, missing, misaligned
    assert L.ssa_select_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 16, None) == _lib.SSA_ERR_WORKSPACE
    assert L.ssa_select_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, None, 1 << 30, None) == _lib.SSA_ERR_NULL
    assert L.ssa_select_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.c_void_p(0x1008), 1 << 30,
                               None) == _lib.SSA_ERR_WORKSPACE
    # dual forward needs sel, both outputs, delta and losses
    st = L.ssa_attn_fwd(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                        FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_NULL
    st = L.ssa_attn_fwd(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_NULL
    st = L.ssa_attn_fwd(ctypes.byref(s), 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_SHAPE
    # backward: sparse stream inputs are required unless FULL_ONLY
    st = L.ssa_attn_bwd(ctypes.byref(s), _lib.SPARSE_ONLY, 1.0, 1.0, FAKE, FAKE, FAKE, None, None,
                        FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_NULL
    st = L.ssa_attn_bwd(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, float("nan"), 1.0, FAKE, FAKE, FAKE,
                        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_SHAPE
    assert L.ssa_status_string(3).decode() == "unsupported configuration"


def test_timing_api_host_side(L):
    from block_sparse_full_ssa_amd import _lib
    assert L.ssa_kernel_count() >= 8
    names = [L.ssa_kernel_name(i).decode() for i in range(L.ssa_kernel_count())]
    assert "fwd_mfma" in names and "select" in names
    assert L.ssa_timing_enable(0) == 0
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.ssa_timing_query(b"select", ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0
    assert L.ssa_timing_query(b"nope", ctypes.byref(ms), ctypes.byref(n)) == _lib.SSA_ERR_SHAPE


def test_fwd_stats_argument_checks(L):
    from block_sparse_full_ssa_amd import _lib
    FAKE = ctypes.c_void_p(1 << 40)
    s = _shape()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]   # q .. losses
    st = L.ssa_attn_fwd_stats(ctypes.byref(s), _lib.SPARSE_ONLY, *args, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_UNSUPPORTED
    st = L.ssa_attn_fwd_stats(ctypes.byref(s), _lib.FULL_ONLY, *args, None, FAKE, None, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_NULL
    st = L.ssa_attn_fwd_stats(ctypes.byref(s), _lib.FULL_ONLY, *args, FAKE, None, None, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_NULL
    bad = _shape(seqlen=250)                      # not a multiple of the block
    st = L.ssa_attn_fwd_stats(ctypes.byref(bad), _lib.FULL_ONLY, *args, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == _lib.SSA_ERR_SHAPE


def test_decode_argument_checks(L):
    from block_sparse_full_ssa_amd import _lib
    FAKE = ctypes.c_void_p(1 << 40)
    s = _shape(seqlen=4096)
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.SPARSE_ONLY, _lib.OP_DECODE) > 0
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.FULL_ONLY, _lib.OP_DECODE) > 0
    assert L.ssa_workspace_size(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, _lib.OP_DECODE) == 0
    ws = 1 << 30
    st = L.ssa_decode(ctypes.byref(s), _lib.DUAL_ACTIVE_FULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                      FAKE, ws, None)
    assert st == _lib.SSA_ERR_UNSUPPORTED
    st = L.ssa_decode(ctypes.byref(s), _lib.SPARSE_ONLY, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                      FAKE, ws, None)
    assert st == _lib.SSA_ERR_NULL                # sparse needs the block means
    st = L.ssa_decode(ctypes.byref(s), _lib.SPARSE_ONLY, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                      FAKE, ws, None)
    assert st == _lib.SSA_ERR_NULL                # ... and sel
    st = L.ssa_decode(ctypes.byref(s), _lib.FULL_ONLY, FAKE, FAKE, FAKE, None, None, FAKE, None, None,
                      FAKE, ws, None)
    assert st == _lib.SSA_ERR_NULL                # pos
    st = L.ssa_decode(ctypes.byref(s), _lib.FULL_ONLY, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None,
                      FAKE, 16, None)
    assert st == _lib.SSA_ERR_WORKSPACE
    assert L.ssa_cache_block_means(ctypes.byref(s), FAKE, FAKE, 3, 2, None) == _lib.SSA_ERR_SHAPE
    assert L.ssa_cache_block_means(ctypes.byref(s), FAKE, FAKE, 0, 4096 // 64 + 1, None) == _lib.SSA_ERR_SHAPE
    assert L.ssa_cache_block_means(ctypes.byref(s), None, FAKE, 0, 1, None) == _lib.SSA_ERR_NULL
    assert L.ssa_cache_block_means(ctypes.byref(s), FAKE, FAKE, 2, 2, None) == _lib.SSA_OK   # nothing to do


def test_probe_argument_checks(L):
    from block_sparse_full_ssa_amd import _lib
    FAKE = ctypes.c_void_p(1 << 40)
    assert L.ssa_probe_mfma(None, 4, 4, None) == _lib.SSA_ERR_NULL
    assert L.ssa_probe_mfma(FAKE, 0, 4, None) == _lib.SSA_ERR_SHAPE
    assert L.ssa_probe_mfma(FAKE, 4, 0, None) == _lib.SSA_ERR_SHAPE
    assert L.ssa_probe_copy(None, FAKE, 16, None) == _lib.SSA_ERR_NULL
    assert L.ssa_probe_copy(FAKE, FAKE, 24, None) == _lib.SSA_ERR_SHAPE
    assert L.ssa_probe_copy(FAKE, FAKE, 0, None) == _lib.SSA_OK      # nothing to launch
    names = [L.ssa_kernel_name(i).decode() for i in range(L.ssa_kernel_count())]
    assert "probe_mfma" in names and "probe_copy" in names


def test_binding_refuses_cpu_tensors():
    import torch
    import block_sparse_full_ssa_amd as ssa
    q = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError):
        ssa.ssa_select_blocks(q, q, 32, 2)
