"""ctypes view of libssa.so (the C interface declared in include/ssa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssa.so")

SSA_OK = 0
SSA_ERR_NULL = 1
SSA_ERR_SHAPE = 2
SSA_ERR_UNSUPPORTED = 3
SSA_ERR_WORKSPACE = 4
SSA_ERR_HIP = 5

SSA_F32 = 0
SSA_BF16 = 1

DUAL_ACTIVE_FULL = 0
DUAL_ACTIVE_SPARSE = 1
FULL_ONLY = 2
SPARSE_ONLY = 3

OP_SELECT = 0
OP_FWD = 1
OP_BWD = 2
OP_DECODE = 3

EXPORTED = (
    "ssa_workspace_size", "ssa_select_blocks", "ssa_attn_fwd", "ssa_attn_fwd_stats", "ssa_attn_bwd",
    "ssa_status_string", "ssa_last_error", "ssa_timing_enable", "ssa_timing_query",
    "ssa_kernel_count", "ssa_kernel_name", "ssa_probe_mfma", "ssa_probe_copy",
    "ssa_cache_block_means", "ssa_decode", "ssa_prefill_workspace_size", "ssa_prefill",
    "ssa_noalloc_scratch_bytes", "ssa_attn_fwd_noalloc", "ssa_probe_atomic", "ssa_probe_lds",
)


class ShapeT(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class SSAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libssa.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python block_sparse_full_ssa_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    shp = ctypes.POINTER(ShapeT)
    L.ssa_workspace_size.argtypes = [shp, i32, i32]
    L.ssa_workspace_size.restype = sz
    L.ssa_select_blocks.argtypes = [shp, vp, vp, vp, vp, sz, vp]
    L.ssa_select_blocks.restype = i32
    L.ssa_attn_fwd.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ssa_attn_fwd.restype = i32
    L.ssa_attn_fwd_stats.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ssa_attn_fwd_stats.restype = i32
    L.ssa_attn_bwd.argtypes = [shp, i32, f32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, sz, vp]
    L.ssa_attn_bwd.restype = i32
    L.ssa_status_string.argtypes = [i32]
    L.ssa_status_string.restype = ctypes.c_char_p
    L.ssa_last_error.argtypes = []
    L.ssa_last_error.restype = ctypes.c_char_p
    L.ssa_timing_enable.argtypes = [i32]
    L.ssa_timing_enable.restype = i32
    L.ssa_timing_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64)]
    L.ssa_timing_query.restype = i32
    L.ssa_kernel_count.argtypes = []
    L.ssa_kernel_count.restype = i32
    L.ssa_kernel_name.argtypes = [i32]
    L.ssa_kernel_name.restype = ctypes.c_char_p
    L.ssa_cache_block_means.argtypes = [shp, vp, vp, i32, i32, vp]
    L.ssa_cache_block_means.restype = i32
    L.ssa_decode.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ssa_decode.restype = i32
    L.ssa_prefill_workspace_size.argtypes = [shp, i32, i32]
    L.ssa_prefill_workspace_size.restype = sz
    L.ssa_prefill.argtypes = [shp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ssa_prefill.restype = i32
    L.ssa_noalloc_scratch_bytes.argtypes = []
    L.ssa_noalloc_scratch_bytes.restype = sz
    L.ssa_attn_fwd_noalloc.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.ssa_attn_fwd_noalloc.restype = i32
    L.ssa_probe_mfma.argtypes = [vp, i32, i32, vp]
    L.ssa_probe_mfma.restype = i32
    L.ssa_probe_copy.argtypes = [vp, vp, sz, vp]
    L.ssa_probe_copy.restype = i32
    L.ssa_probe_atomic.argtypes = [vp, ctypes.c_int64, i32, i32, vp]
    L.ssa_probe_atomic.restype = i32
    L.ssa_probe_lds.argtypes = [vp, i32, i32, i32, vp]
    L.ssa_probe_lds.restype = i32
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != SSA_OK:
        L = lib()
        detail = L.ssa_last_error().decode() or L.ssa_status_string(status).decode()
        raise SSAError(status, where, detail)
