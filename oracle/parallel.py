"""Process-pool driver of the oracle over one (batch, KV head) unit.

TEST INFRASTRUCTURE ONLY (the full-size parity tests and the benchmark's
CPU-baseline leg).  It shares no code with the HIP path.

A unit is the G query heads that share one KV head, with that KV head's keys
and values.  Units are independent in the forward and the backward (dk and dv
sum only over the unit's own query heads), so one unit at a layer's real
sequence length is the oracle's share of that layer.  The driver cuts the
unit's query rows into (head, row chunk) tasks and runs, for each task, the
oracle's own row functions in order: selection (select_rows), both streams
(attend_rows), the stream gradients (stream_grads, with the layer's element
count M) and the row backward (_bwd_rows).  It adds no arithmetic of its own
except summing the workers' dk / dv contributions.

Inputs and outputs live in shared memory; each worker process runs one BLAS
thread, so the pool's size is the number of cores used.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import threading
import time
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import shared_memory

import numpy as np

from . import ssa_oracle as O

_CHUNK = 256
_START_TIMEOUT = 300.0

# worker-side state (set by _init in each worker process)
_W = {}


def _attach(spec):
    arrays, handles = {}, []
    for name, (shm_name, shape, dtype) in spec.items():
        h = shared_memory.SharedMemory(name=shm_name)
        handles.append(h)
        arrays[name] = np.ndarray(shape, dtype=dtype, buffer=h.buf)
    return arrays, handles


def _init(spec, cfg, counter, barrier):
    import threadpoolctl

    threadpoolctl.threadpool_limits(1)
    arrays, handles = _attach(spec)
    with counter.get_lock():
        wid = counter.value
        counter.value += 1
    _W.update(arrays=arrays, handles=handles, cfg=cfg, wid=wid,
              mu=O.block_means(arrays["k"][None, None], cfg["block"])[0, 0])
    barrier.wait(timeout=_START_TIMEOUT)


def _task(args):
    h, t0, t1 = args
    A, cfg = _W["arrays"], _W["cfg"]
    mode, block, K, scale = cfg["mode"], cfg["block"], cfg["top_k"], cfg["scale"]
    t_idx = np.arange(t0, t1)
    q_h, k_c, v_c = A["q"][h], A["k"], A["v"]
    if mode == O.FULL_ONLY:
        sel_rows = None
    elif "sel_in" in A:
        sel_rows = A["sel_in"][h, t0:t1]
    else:
        sel_rows, margin = O.select_rows(q_h[t_idx], t_idx, _W["mu"], block, K)
        A["sel"][h, t0:t1] = sel_rows
        A["margin"][h, t0:t1] = margin
    want_f, want_s = mode != O.SPARSE_ONLY, mode != O.FULL_ONLY
    o = O.attend_rows(q_h[t_idx], t_idx, k_c, v_c, sel_rows, block, scale, want_f, want_s)
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta"):
        if key in o:
            A[key][h, t0:t1] = o[key]
    if not cfg["backward"]:
        return
    dout = A["dout"][h, t0:t1] if "dout" in A else None
    g_f, g_s = O.stream_grads(mode, dout, o.get("h_full"), o.get("h_sparse"), cfg["w_sparsity"],
                              cfg["w_commit"], M=cfg["M"])
    wid = _W["wid"]
    # tasks own disjoint rows of dq (zeroed), and each worker its own dk / dv slot
    O._bwd_rows(q_h, k_c, v_c, t_idx, sel_rows, block, scale, g_f, g_s, o.get("h_full"), o.get("h_sparse"),
                A["dq"][h], A["dk_w"][wid], A["dv_w"][wid])


def _ready():
    return True


def pool_size() -> int:
    """Cores this process may run on (at most 16, the CPU share of one GPU machine)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def unit_step(q_u, k_c, v_c, block, top_k, scale, mode, dout_u=None, sel_u=None, backward=True,
              w_sparsity=1.0, w_commit=1.0, M=None, workers=None):
    """Selection (unless ``sel_u`` is given), both streams and, with
    ``backward``, dq / dk / dv of one unit, on a process pool.

    q_u [G, N, d], k_c and v_c [N, d] (float64), dout_u [G, N, d] or None,
    sel_u [G, N, top_k] or None.  ``M`` is the element count of the whole
    layer the unit belongs to (the alignment losses are means over it).
    Returns a dict with the arrays of the unit (sel and margin when selected
    here, h_*, lse_*, delta, dq [G, N, d], dk and dv [N, d]), plus "seconds"
    (the pool's wall time, setup excluded) and "workers".
    """
    G, N, d = q_u.shape
    W = workers or pool_size()
    M = M if M is not None else q_u.size
    want_f, want_s = mode != O.SPARSE_ONLY, mode != O.FULL_ONLY
    shapes = {"q": ((G, N, d), np.float64), "k": ((N, d), np.float64), "v": ((N, d), np.float64)}
    if dout_u is not None:
        shapes["dout"] = ((G, N, d), np.float64)
    if sel_u is not None:
        shapes["sel_in"] = ((G, N, top_k), np.int32)
    elif mode != O.FULL_ONLY:
        shapes["sel"] = ((G, N, top_k), np.int32)
        shapes["margin"] = ((G, N), np.float64)
    if want_f:
        shapes["h_full"] = ((G, N, d), np.float64)
        shapes["lse_full"] = ((G, N), np.float64)
    if want_s:
        shapes["h_sparse"] = ((G, N, d), np.float64)
        shapes["lse_sparse"] = ((G, N), np.float64)
    if want_f and want_s:
        shapes["delta"] = ((G, N), np.float64)
    if backward:
        shapes["dq"] = ((G, N, d), np.float64)
        shapes["dk_w"] = ((W, N, d), np.float64)
        shapes["dv_w"] = ((W, N, d), np.float64)
    handles, spec, arrays = [], {}, {}
    try:
        for name, (shape, dtype) in shapes.items():
            nbytes = max(1, int(np.prod(shape)) * np.dtype(dtype).itemsize)
            h = shared_memory.SharedMemory(create=True, size=nbytes)
            handles.append(h)
            spec[name] = (h.name, shape, dtype)
            arrays[name] = np.ndarray(shape, dtype=dtype, buffer=h.buf)
            if name in ("dq", "dk_w", "dv_w"):
                arrays[name][...] = 0.0
        arrays["q"][...] = q_u
        arrays["k"][...] = k_c
        arrays["v"][...] = v_c
        if dout_u is not None:
            arrays["dout"][...] = dout_u
        if sel_u is not None:
            arrays["sel_in"][...] = sel_u
        cfg = dict(mode=mode, block=block, top_k=top_k, scale=scale, backward=backward, M=M,
                   w_sparsity=w_sparsity, w_commit=w_commit)
        # longest rows first: chunks late in the sequence see the most keys
        tasks = [(h, t0, min(N, t0 + _CHUNK)) for t0 in range(0, N, _CHUNK) for h in range(G)]
        tasks.sort(key=lambda x: -x[2])
        # fresh worker processes (spawn): the caller may hold GPU state that a
        # fork must not inherit; a worker that dies breaks the pool and raises
        ctx = mp.get_context("spawn")
        counter = ctx.Value("i", 0)
        barrier = ctx.Barrier(W + 1)
        with ProcessPoolExecutor(W, mp_context=ctx, initializer=_init,
                                 initargs=(spec, cfg, counter, barrier)) as pool:
            futs = [pool.submit(_ready) for _ in range(W)]   # one task each starts W workers
            try:
                barrier.wait(timeout=_START_TIMEOUT)   # all attached before timing
            except threading.BrokenBarrierError:
                for f in futs:
                    f.result(timeout=1)                 # the worker's own error, if it has one
                raise RuntimeError("oracle worker processes did not start")
            t0 = time.perf_counter()
            futs += [pool.submit(_task, t) for t in tasks]
            for f in futs:
                f.result()
            seconds = time.perf_counter() - t0
        out = {name: np.array(arr) for name, arr in arrays.items()
               if name not in ("q", "k", "v", "dout", "sel_in", "dk_w", "dv_w")}
        if backward:
            out["dk"] = arrays["dk_w"].sum(axis=0)
            out["dv"] = arrays["dv_w"].sum(axis=0)
        out["seconds"] = seconds
        out["workers"] = W
        return out
    finally:
        arrays.clear()
        for h in handles:
            h.close()
            h.unlink()
