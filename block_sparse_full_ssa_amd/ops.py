"""Torch-facing binding of libssa: argument marshalling only.

Each function checks tensor placement, allocates its outputs and workspace
with torch on the inputs' device, and calls the C entry point of the same
name on torch's current stream.  Every step of the computation runs in the
library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY  # noqa: F401

_DT = {torch.float32: _lib.SSA_F32, torch.bfloat16: _lib.SSA_BF16}


def make_shape(q: torch.Tensor, k: torch.Tensor, block: int, top_k: int,
               scale: Optional[float] = None) -> _lib.ShapeT:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DT or k.dtype != q.dtype:
        raise ValueError("q and k must both be float32 or bfloat16")
    return _lib.ShapeT(B, Hq, Hq // Hkv, N, d, int(block), int(top_k),
                       0.0 if scale is None else float(scale), _DT[q.dtype])


def _check_layer(q, k, v, sel, top_k: int, need_sel: bool) -> None:
    """Shapes and dtypes the kernels index by: v like k, sel int32 [B, Hq, N, top_k]."""
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError(f"v {tuple(v.shape)} {v.dtype} must match k {tuple(k.shape)} {k.dtype}")
    if sel is None:
        if need_sel:
            raise ValueError("sel is required for modes with the sparse stream")
        return
    B, Hq, N, _ = q.shape
    if sel.dtype != torch.int32 or tuple(sel.shape) != (B, Hq, N, int(top_k)):
        raise ValueError(f"sel must be int32 {(B, Hq, N, int(top_k))}, got {sel.dtype} {tuple(sel.shape)}")


def _check_like(name: str, t: Optional[torch.Tensor], shape, dtype, required: bool) -> None:
    if t is None:
        if required:
            raise ValueError(f"{name} is required in this mode")
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_check(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libssa works on GPU tensors")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        dev = t.device if dev is None else dev
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(shape, mode, op, dev) -> Tuple[Optional[torch.Tensor], int, int]:
    n = _lib.lib().ssa_workspace_size(ctypes.byref(shape), mode, op)
    if n == 0:
        return None, 0, 0
    buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 256
    return buf, buf.data_ptr() + off, n


def ssa_select_blocks(q: torch.Tensor, k: torch.Tensor, block: int, top_k: int) -> torch.Tensor:
    """Selected key blocks [B, Hq, N, top_k] int32, ascending, -1 padded."""
    dev = _dev_check(q, k)
    shape = make_shape(q, k, block, top_k)
    B, Hq, N, _ = q.shape
    sel = torch.empty(B, Hq, N, top_k, dtype=torch.int32, device=dev)
    ws, wp, wn = _workspace(shape, 0, _lib.OP_SELECT, dev)
    st = _lib.lib().ssa_select_blocks(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(sel),
                                      ctypes.c_void_p(wp), wn, _stream(dev))
    _lib.check(st, "ssa_select_blocks")
    return sel


def ssa_attn_fwd(q, k, v, sel, block: int, top_k: int, mode: int = DUAL_ACTIVE_FULL,
                 scale: Optional[float] = None, want_lse: bool = True,
                 stats: bool = False) -> Dict[str, torch.Tensor]:
    """Forward of one SSA layer; returns the outputs the mode defines.

    With ``stats`` (modes with the full stream) it calls ssa_attn_fwd_stats and
    also returns the full stream's per-row ``sink_mass`` and ``entropy`` and
    their per-head means ``head_stats`` [B, Hq, 2]."""
    dev = _dev_check(q, k, v, sel)
    shape = make_shape(q, k, block, top_k, scale)
    _check_layer(q, k, v, sel, top_k, mode != FULL_ONLY)
    B, Hq, N, d = q.shape
    dual = mode in (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE)
    out: Dict[str, torch.Tensor] = {}
    f32 = dict(dtype=torch.float32, device=dev)
    if mode != SPARSE_ONLY:
        out["h_full"] = torch.empty_like(q)
        if want_lse:
            out["lse_full"] = torch.empty(B, Hq, N, **f32)
    if mode != FULL_ONLY:
        out["h_sparse"] = torch.empty_like(q)
        if want_lse:
            out["lse_sparse"] = torch.empty(B, Hq, N, **f32)
    if dual:
        out["delta"] = torch.empty(B, Hq, N, **f32)
        out["losses"] = torch.empty(2, **f32)
    ws, wp, wn = _workspace(shape, mode, _lib.OP_FWD, dev)
    common = (ctypes.byref(shape), int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
              _ptr(out.get("h_full")), _ptr(out.get("h_sparse")), _ptr(out.get("lse_full")),
              _ptr(out.get("lse_sparse")), _ptr(out.get("delta")), _ptr(out.get("losses")))
    if stats:
        out["sink_mass"] = torch.empty(B, Hq, N, **f32)
        out["entropy"] = torch.empty(B, Hq, N, **f32)
        out["head_stats"] = torch.empty(B, Hq, 2, **f32)
        st = _lib.lib().ssa_attn_fwd_stats(*common, _ptr(out["sink_mass"]), _ptr(out["entropy"]),
                                           _ptr(out["head_stats"]), ctypes.c_void_p(wp), wn, _stream(dev))
        _lib.check(st, "ssa_attn_fwd_stats")
    else:
        st = _lib.lib().ssa_attn_fwd(*common, ctypes.c_void_p(wp), wn, _stream(dev))
        _lib.check(st, "ssa_attn_fwd")
    if ws is not None:
        out["_ws"] = ws   # keeps the workspace alive until the caller drops the dict
    return out


def ssa_attn_fwd_noalloc(q, k, v, sel, block: int, top_k: int, mode: int = DUAL_ACTIVE_FULL,
                         scale: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """ssa_attn_fwd with the library's static per-device workspace instead of
    a caller buffer (the C entry point allocates nothing; this wrapper only
    allocates the outputs)."""
    dev = _dev_check(q, k, v, sel)
    shape = make_shape(q, k, block, top_k, scale)
    _check_layer(q, k, v, sel, top_k, mode != FULL_ONLY)
    B, Hq, N, d = q.shape
    f32 = dict(dtype=torch.float32, device=dev)
    out: Dict[str, torch.Tensor] = {}
    if mode != SPARSE_ONLY:
        out["h_full"] = torch.empty_like(q)
        out["lse_full"] = torch.empty(B, Hq, N, **f32)
    if mode != FULL_ONLY:
        out["h_sparse"] = torch.empty_like(q)
        out["lse_sparse"] = torch.empty(B, Hq, N, **f32)
    if mode in (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE):
        out["delta"] = torch.empty(B, Hq, N, **f32)
        out["losses"] = torch.empty(2, **f32)
    st = _lib.lib().ssa_attn_fwd_noalloc(
        ctypes.byref(shape), int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out.get("h_full")),
        _ptr(out.get("h_sparse")), _ptr(out.get("lse_full")), _ptr(out.get("lse_sparse")), _ptr(out.get("delta")),
        _ptr(out.get("losses")), _stream(dev))
    _lib.check(st, "ssa_attn_fwd_noalloc")
    return out


def ssa_attn_bwd(q, k, v, sel, fwd: Dict[str, torch.Tensor], d_out: Optional[torch.Tensor],
                 block: int, top_k: int, mode: int = DUAL_ACTIVE_FULL, w_sparsity: float = 1.0,
                 w_commit: float = 1.0, scale: Optional[float] = None):
    """(dq, dk, dv) of one SSA layer from the forward's saved outputs."""
    dev = _dev_check(q, k, v, sel, d_out, *(fwd.get(n) for n in ("h_full", "h_sparse", "lse_full", "lse_sparse")))
    shape = make_shape(q, k, block, top_k, scale)
    _check_layer(q, k, v, sel, top_k, mode != FULL_ONLY)
    rows = tuple(q.shape[:3])
    has_full, has_sparse = mode != SPARSE_ONLY, mode != FULL_ONLY
    _check_like("d_out", d_out, q.shape, q.dtype, False)
    _check_like("fwd['h_full']", fwd.get("h_full"), q.shape, q.dtype, has_full)
    _check_like("fwd['lse_full']", fwd.get("lse_full"), rows, torch.float32, has_full)
    _check_like("fwd['h_sparse']", fwd.get("h_sparse"), q.shape, q.dtype, has_sparse)
    _check_like("fwd['lse_sparse']", fwd.get("lse_sparse"), rows, torch.float32, has_sparse)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws, wp, wn = _workspace(shape, mode, _lib.OP_BWD, dev)
    st = _lib.lib().ssa_attn_bwd(
        ctypes.byref(shape), int(mode), float(w_sparsity), float(w_commit),
        _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(fwd.get("h_full")), _ptr(fwd.get("h_sparse")),
        _ptr(fwd.get("lse_full")), _ptr(fwd.get("lse_sparse")), _ptr(d_out),
        _ptr(dq), _ptr(dk), _ptr(dv), ctypes.c_void_p(wp), wn, _stream(dev))
    _lib.check(st, "ssa_attn_bwd")
    del ws
    return dq, dk, dv


def timing_enable(on: bool = True) -> None:
    _lib.check(_lib.lib().ssa_timing_enable(1 if on else 0), "ssa_timing_enable")


def timing_query(kernel: str) -> Tuple[float, int]:
    """(total milliseconds, launches) of one library kernel since timing_enable."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _lib.check(_lib.lib().ssa_timing_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)),
               "ssa_timing_query")
    return ms.value, n.value


def kernel_names():
    L = _lib.lib()
    return [L.ssa_kernel_name(i).decode() for i in range(L.ssa_kernel_count())]


def ssa_probe_mfma(sink: torch.Tensor, blocks: int, iters: int) -> None:
    """Enqueue the dense bf16 matrix-core probe (blocks * 16 * iters * 32768 flops).

    ``sink`` is a CUDA float32 tensor of at least blocks * 256 elements."""
    if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("sink must be a CUDA float32 tensor of >= blocks * 256 elements")
    _lib.check(_lib.lib().ssa_probe_mfma(_ptr(sink), int(blocks), int(iters), _stream(sink.device)),
               "ssa_probe_mfma")


def ssa_probe_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Enqueue the plain device copy probe of src's bytes into dst."""
    if not (src.is_cuda and dst.is_cuda) or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous CUDA tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _lib.check(_lib.lib().ssa_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device)), "ssa_probe_copy")


def ssa_probe_atomic(buf: torch.Tensor, blocks: int, iters: int) -> None:
    """Enqueue the fp32 atomic probe on ``buf`` (CUDA float32, a multiple of
    4096 elements): blocks * iters * 16 KiB of atomic adds."""
    if not buf.is_cuda or buf.dtype != torch.float32 or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA float32 tensor")
    _lib.check(_lib.lib().ssa_probe_atomic(_ptr(buf), buf.numel(), int(blocks), int(iters), _stream(buf.device)),
               "ssa_probe_atomic")


def ssa_probe_lds(sink: torch.Tensor, blocks: int, iters: int, mode: int) -> None:
    """Enqueue the LDS read probe (mode 0: 16-byte reads, 1: transposing 8-byte reads)."""
    if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("sink must be a CUDA float32 tensor of >= blocks * 256 elements")
    _lib.check(_lib.lib().ssa_probe_lds(_ptr(sink), int(blocks), int(iters), int(mode), _stream(sink.device)),
               "ssa_probe_lds")


def _cache_shape(q: torch.Tensor, k_cache: torch.Tensor, block: int, top_k: int,
                 scale: Optional[float]) -> _lib.ShapeT:
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k_cache [B, Hkv, L, d]")
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d or Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if q.dtype not in _DT or k_cache.dtype != q.dtype:
        raise ValueError("q and the caches must both be float32 or bfloat16")
    return _lib.ShapeT(B, Hq, Hq // Hkv, L, d, int(block), int(top_k),
                       0.0 if scale is None else float(scale), _DT[q.dtype])


def ssa_cache_block_means(k_cache: torch.Tensor, mu_cache: torch.Tensor, block: int, block_begin: int,
                          block_end: int) -> None:
    """mu_cache[:, :, j] = mean of k_cache's keys of block j, for block_begin <= j < block_end.

    k_cache [B, Hkv, L, d]; mu_cache [B, Hkv, L / block, d] float32 (both CUDA)."""
    dev = _dev_check(k_cache, mu_cache)
    B, Hkv, L, d = k_cache.shape
    if mu_cache.dtype != torch.float32 or tuple(mu_cache.shape) != (B, Hkv, L // block, d):
        raise ValueError("mu_cache must be float32 [B, Hkv, L / block, d]")
    shape = _lib.ShapeT(B, Hkv, 1, L, d, int(block), 1, 0.0, _DT[k_cache.dtype])
    _lib.check(_lib.lib().ssa_cache_block_means(ctypes.byref(shape), _ptr(k_cache), _ptr(mu_cache),
                                                int(block_begin), int(block_end), _stream(dev)),
               "ssa_cache_block_means")


def ssa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, mu_cache: Optional[torch.Tensor],
               pos: torch.Tensor, block: int, top_k: int, mode: int = SPARSE_ONLY,
               scale: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """One decode step: q [B, Hq, d] of the tokens at positions pos [B] (int32,
    CUDA) over the caches.  Returns h [B, Hq, d], lse [B, Hq] and, for
    SPARSE_ONLY, the selection sel [B, Hq, top_k]."""
    dev = _dev_check(q, k_cache, v_cache, mu_cache, pos)
    if pos.dtype != torch.int32 or pos.numel() != q.shape[0]:
        raise ValueError("pos must be int32 [B]")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    shape = _cache_shape(q, k_cache, block, top_k, scale)
    B, Hq, d = q.shape
    out = {"h": torch.empty_like(q), "lse": torch.empty(B, Hq, dtype=torch.float32, device=dev)}
    if mode == SPARSE_ONLY:
        out["sel"] = torch.empty(B, Hq, int(top_k), dtype=torch.int32, device=dev)
    ws, wp, wn = _workspace(shape, mode, _lib.OP_DECODE, dev)
    st = _lib.lib().ssa_decode(ctypes.byref(shape), int(mode), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(mu_cache), _ptr(pos), _ptr(out["h"]), _ptr(out["lse"]), _ptr(out.get("sel")),
                               ctypes.c_void_p(wp), wn, _stream(dev))
    _lib.check(st, "ssa_decode")
    if ws is not None:
        out["_ws"] = ws
    return out


def ssa_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, mu_cache: Optional[torch.Tensor],
                pos0: int, block: int, top_k: int, mode: int = SPARSE_ONLY,
                scale: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """A prefill chunk: q [B, Hq, C, d] of the tokens at positions pos0 .. pos0 + C - 1
    over the caches [B, Hkv, L, d] (their keys and values already written).
    Returns h [B, Hq, C, d], lse [B, Hq, C] and, for SPARSE_ONLY, sel [B, Hq, C, top_k]."""
    dev = _dev_check(q, k_cache, v_cache, mu_cache)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, C, d] and k_cache [B, Hkv, L, d]")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    B, Hq, C, d = q.shape
    shape = _cache_shape(q[:, :, 0], k_cache, block, top_k, scale)
    out = {"h": torch.empty_like(q), "lse": torch.empty(B, Hq, C, dtype=torch.float32, device=dev)}
    if mode == SPARSE_ONLY:
        out["sel"] = torch.empty(B, Hq, C, int(top_k), dtype=torch.int32, device=dev)
    L = _lib.lib()
    n = L.ssa_prefill_workspace_size(ctypes.byref(shape), int(mode), int(C))
    ws, wp = None, 0
    if n:
        ws = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        wp = ws.data_ptr() + (-ws.data_ptr()) % 256
    st = L.ssa_prefill(ctypes.byref(shape), int(mode), _ptr(q), int(pos0), int(C), _ptr(k_cache), _ptr(v_cache),
                       _ptr(mu_cache), _ptr(out["h"]), _ptr(out["lse"]), _ptr(out.get("sel")),
                       ctypes.c_void_p(wp), n, _stream(dev))
    _lib.check(st, "ssa_prefill")
    if ws is not None:
        out["_ws"] = ws
    return out
