"""Throughput of one SSA training step of attention on one MI355X.

A step is the whole hot path over one batch of the 16K-context training
layer (B=2, 32 query / 8 KV heads, N=16384, d=128, bf16, block 64, top_k 16
by default): block selection, the dual-stream forward (full and sparse
outputs, delta, alignment losses) and the backward with the active stream
drawn 50/50 per step from the seed.  Inputs are synthetic and resident in
HBM before timing starts.

Reported (one JSON line):
  value / ms_per_step   algorithmic TFLOP/s of the step, wall clock over the
                        timed steps with the library's event timing off;
  roofline              the dominant kernel: its algorithmic flops per launch
                        over its average launch time, from HIP events recorded
                        on the launch stream in a second pass of as many steps;
  top_k_sweep           the step at top_k 4, 8, 16, 32;
  full_only             FULL_ONLY fwd+bwd, the full stream alone (14 d P_full B Hq);
  sparse_fwd_speedup    per top_k, t(FULL_ONLY fwd) / t(SPARSE_ONLY fwd) next to
                        P_full / P_sparse and N / (top_k block), with the HBM
                        rates of the selection and the sparse-only forward
                        against their compulsory bytes;
  sparse_only_train     SPARSE_ONLY fwd+bwd (pure sparse training) against
                        FULL_ONLY fwd+bwd;
  long_n64k_sinks       the 64K-context layer with planted sinks: selection +
                        dual forward;
  multilayer_b4_n8k_l4  four layers forward then backward, 10 timed steps;
  decode_128k           sparse vs full decode and prefill over a 128K cache;
  cpu_baseline          the fp64 oracle on the host's cores: one whole
                        (batch, KV head) unit of the training step, scaled by
                        the B * Hkv units of the layer to seconds per step.

Algorithmic work (FlashAttention convention, recompute included): per causal
(query, key) pair 4d flops forward and 10d backward, counted for the full
stream (P_full = N(N+1)/2 pairs per head) and for the sparse stream
(P_sparse = sum over queries of the selected causal keys), i.e.
14 d (P_full + P_sparse) B Hq per step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def pairs(N: int, block: int, K: int):
    """(P_full, P_sparse) causal pairs per head for the stated selection."""
    nb = N // block
    p_full = N * (N + 1) // 2
    # query block i keeps min(K-1, i) earlier full blocks plus its own causal part
    p_sparse = block * block * sum(min(i, K - 1) for i in range(nb)) + nb * block * (block + 1) // 2
    return p_full, p_sparse


def algorithmic_flops_per_launch(d, pf, ps, heads):
    """Algorithmic flops that one launch of each bf16 matrix kernel performs
    (FlashAttention convention: per causal pair 4d forward, 10d backward).

    Training step (both streams):
    fwd_mfma:   both streams' forward, 4d (P_full + P_sparse);
    bwd_mfma:   full stream dK and dV with the S and dP they recompute, 8d P_full;
    bwd_dq:     dQ of both streams, 2d (P_full + P_sparse) (the full stream's
                S / dP recompute is extra; the sparse stream's dS comes in);
    bwd_sparse: the sparse stream's S, dP, dK and dV, 8d P_sparse;
    sparse_part: the sparse-only forward, 4d P_sparse.
    The kernels' shares add up to 14 d (P_full + P_sparse).
    """
    return {"fwd_mfma": 4.0 * d * (pf + ps) * heads, "bwd_mfma": 8.0 * d * pf * heads,
            "bwd_dq": 2.0 * d * (pf + ps) * heads, "bwd_sparse": 8.0 * d * ps * heads,
            "sparse_part": 4.0 * d * ps * heads}


def profile_record(name, kernel, workload, top_k):
    """The record of ``kernel`` in the committed rocprofv3 summary
    ``profiles/<name>.json``, or None when there is none for this workload or
    the kernel's source changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}/{workload}/top_k={top_k}")
    if not rec:
        return None
    src = os.path.join(ROOT, "block_sparse_full_ssa_amd", "csrc", rec["source"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec


def measured_traffic(kernel, workload, top_k):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated by a plain copy), or None."""
    rec = profile_record("hbm_traffic", kernel, workload, top_k)
    return rec["bytes_per_launch"] if rec else None


def matrix_pipe_use(kernels, workload, top_k):
    """Per matrix kernel, rocprofv3's MfmaUtil (matrix pipes busy over active
    cycles), the executed bf16 matrix flops and the clock, from the committed
    counter summary; None for a kernel whose source changed since."""
    out = {}
    for kid in kernels:
        rec = profile_record("mfma_util", kid, workload, top_k)
        out[kid] = None if rec is None else {k: rec[k] for k in ("mfma_util_pct", "clock_ghz", "executed_bf16_flops")}
    return out


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train_b2_h32_n16k")
    ap.add_argument("--top-k", type=int, default=None)
    ap.add_argument("--seqlen", type=int, default=None, help="override N (experiments only)")
    ap.add_argument("--batch", type=int, default=None, help="override B (experiments only)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true", help="skip the top_k sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the 128K-cache decode leg")
    ap.add_argument("--no-single-stream", action="store_true",
                    help="skip the FULL_ONLY / SPARSE_ONLY measurements")
    ap.add_argument("--no-other-layers", action="store_true",
                    help="skip the 64K-context layer and the four-layer slice")
    return ap.parse_args()


def train_steps(ssa, q, k, v, dout, block, K, modes):
    """One training step per mode in ``modes``: select + dual fwd + bwd."""
    out = None
    for mode in modes:
        sel = ssa.ssa_select_blocks(q, k, block, K)
        fwd = ssa.ssa_attn_fwd(q, k, v, sel, block, K, mode)
        out = ssa.ssa_attn_bwd(q, k, v, sel, fwd, dout, block, K, mode)
    return out


def wall_ms(fn, calls, warm=1):
    """Wall-clock milliseconds per call of ``fn`` (GPU work included), after warm-up."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / calls


def kernel_times(ssa, fn):
    """Per-kernel device times of ``fn()`` from the library's HIP events
    (recorded on each kernel's launch stream): {name: (total ms, launches)}."""
    import torch

    torch.cuda.synchronize()
    ssa.timing_enable(True)
    fn()
    torch.cuda.synchronize()
    res = {}
    for name in ssa.kernel_names():
        ms, n = ssa.timing_query(name)
        if n:
            res[name] = (ms, n)
    ssa.timing_enable(False)
    return res


def hbm_rates(ssa, q, k, v, sel, block, K, reps):
    """HBM rates of the two HBM-bound steps (a2 selection, a8 sparse-only
    forward), device time from the library's events, against the 8 TB/s peak.

    Compulsory bytes (what the step must move at least): selection reads q
    and k and writes sel; the sparse-only forward reads q, k, v and sel and
    writes h_sparse and lse_sparse.  The implementation's bytes are given
    apart: the selection also writes and reads the block means; the
    sparse-only forward gathers the query row of every selected (row, block)
    pair into its key block's bucket, and writes and reads one partial per
    pair (d bf16 values and an fp32 log-sum-exp)."""
    B, Hq, N, d = q.shape
    nb = N // block
    el = q.element_size()

    def dev_ms(fn, names):
        t = kernel_times(ssa, lambda: [fn() for _ in range(reps)])
        return sum(t[n][0] for n in names if n in t) / reps

    ms_sel = dev_ms(lambda: ssa.ssa_select_blocks(q, k, block, K), ("block_mean", "select"))
    ms_sp = dev_ms(lambda: ssa.ssa_attn_fwd(q, k, v, sel, block, K, ssa.SPARSE_ONLY),
                   ("bucket", "sparse_part", "sparse_merge"))
    rows = q.numel() // d
    sel_bytes = rows * K * 4
    mu_bytes = B * k.shape[1] * nb * d * 4
    c_sel = (q.numel() + k.numel()) * el + sel_bytes
    c_sp = (q.numel() + k.numel() + v.numel()) * el + sel_bytes + q.numel() * el + rows * 4
    entries = B * Hq * sum(min(K, t // block + 1) for t in range(N))
    i_sel = c_sel + 2 * mu_bytes
    i_sp = c_sp + entries * d * el + 2 * entries * (d * 2 + 4)

    def rate(b, ms):
        return round(b / (ms / 1e3) / 1e9, 1)

    return {"select_ms": round(ms_sel, 4), "select_bytes": c_sel, "select_GBps": rate(c_sel, ms_sel),
            "select_frac_of_hbm": round(rate(c_sel, ms_sel) / HBM_PEAK_GBS, 4),
            "sparse_fwd_ms": round(ms_sp, 4), "sparse_fwd_bytes": c_sp, "sparse_fwd_GBps": rate(c_sp, ms_sp),
            "sparse_fwd_frac_of_hbm": round(rate(c_sp, ms_sp) / HBM_PEAK_GBS, 4),
            "implementation": {"select_bytes": i_sel, "select_GBps": rate(i_sel, ms_sel),
                               "sparse_fwd_bytes": i_sp, "sparse_fwd_GBps": rate(i_sp, ms_sp)},
            "bytes": "compulsory: select q + k read, sel written; sparse-only fwd q, k, v, sel read, "
                     "h_sparse + lse_sparse written"}


def single_stream(ssa, q, k, v, dout, block, K0, ks, reps):
    """FULL_ONLY fwd+bwd (14 d P_full B Hq per step), and per top_k the
    sparse-stream forward speedup and the SPARSE_ONLY fwd+bwd step."""
    B, Hq, N, d = q.shape
    pf, _ = pairs(N, block, K0)

    def full_fwd():
        return ssa.ssa_attn_fwd(q, k, v, None, block, K0, ssa.FULL_ONLY)

    def full_step():
        f = full_fwd()
        ssa.ssa_attn_bwd(q, k, v, None, f, dout, block, K0, ssa.FULL_ONLY)

    ms_full = wall_ms(full_step, reps)
    ms_full_fwd = wall_ms(full_fwd, reps)
    fl = 14.0 * d * pf * B * Hq
    out = {"full_only": {"ms_per_step": round(ms_full, 3), "TFLOP/s": round(fl / (ms_full / 1e3) / 1e12, 2),
                         "frac_of_bf16_peak": round(fl / (ms_full / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "fwd_ms": round(ms_full_fwd, 3), "bwd_ms": round(ms_full - ms_full_fwd, 3),
                         "fwd_frac_of_bf16_peak": round(4.0 * d * pf * B * Hq / (ms_full_fwd / 1e3) / 1e12
                                                        / MFMA_BF16_PEAK_TFLOPS, 4),
                         "ms_at_half_peak": round(fl / (0.5 * MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3, 3),
                         "step": "FULL_ONLY fwd + bwd, 14 d P_full B Hq flops"}}
    sp, train = {}, {}
    for kk in ks:
        sel = ssa.ssa_select_blocks(q, k, block, kk)
        ms_sel = wall_ms(lambda: ssa.ssa_select_blocks(q, k, block, kk), reps)

        def sp_fwd():
            return ssa.ssa_attn_fwd(q, k, v, sel, block, kk, ssa.SPARSE_ONLY)

        def sp_step():
            f = sp_fwd()
            ssa.ssa_attn_bwd(q, k, v, sel, f, dout, block, kk, ssa.SPARSE_ONLY)

        ms_sp = wall_ms(sp_fwd, reps)
        ms_sp_step = wall_ms(sp_step, reps)
        a, b = pairs(N, block, kk)
        sp[str(kk)] = {"sparse_only_fwd_ms": round(ms_sp, 3), "select_ms": round(ms_sel, 3),
                       "speedup": round(ms_full_fwd / ms_sp, 2),
                       "speedup_incl_select": round(ms_full_fwd / (ms_sp + ms_sel), 2),
                       "P_full/P_sparse": round(a / b, 2), "N/(K*block)": round(N / (kk * block), 2),
                       "hbm": hbm_rates(ssa, q, k, v, sel, block, kk, reps)}
        fl_sp = 14.0 * d * b * B * Hq
        train[str(kk)] = {"sparse_only_fwd_bwd_ms": round(ms_sp_step, 3),
                          "incl_select_ms": round(ms_sp_step + ms_sel, 3),
                          "speedup_vs_full_only": round(ms_full / ms_sp_step, 2),
                          "speedup_incl_select": round(ms_full / (ms_sp_step + ms_sel), 2),
                          "TFLOP/s": round(fl_sp / (ms_sp_step / 1e3) / 1e12, 2),
                          "P_full/P_sparse": round(a / b, 2)}
        del sel
    out["sparse_fwd_speedup"] = sp
    out["sparse_only_train"] = {"per_top_k": train,
                                "step": "SPARSE_ONLY fwd + bwd (pure sparse training) against FULL_ONLY fwd + bwd"}

    # full-stream diagnostics (sink-block mass, entropy, per-head means) in the
    # forward pass: cost over the plain FULL_ONLY forward, and the head means
    ms_stats = wall_ms(lambda: ssa.ssa_attn_fwd(q, k, v, None, block, K0, ssa.FULL_ONLY, stats=True), reps)
    st = ssa.ssa_attn_fwd(q, k, v, None, block, K0, ssa.FULL_ONLY, stats=True)["head_stats"]
    out["full_stats"] = {"fwd_ms": round(ms_stats, 3), "overhead": round(ms_stats / ms_full_fwd - 1.0, 4),
                         "mean_sink_mass": round(float(st[..., 0].mean()), 5),
                         "mean_entropy_nats": round(float(st[..., 1].mean()), 4)}
    return out


def long_layer(ssa, dev, seed, reps):
    """The 64K-context layer with four planted sinks (B=1, 16/4 heads, block 64,
    top_k 32): selection + dual forward (sparse stream active, full counterpart
    and delta), inputs drawn on the GPU."""
    import ssa_inputs as si

    wl = si.WORKLOADS["long_n64k_sinks"]
    q, k, v, _ = si.draw_qkv(wl, seed, device=str(dev))
    K, blk = wl.top_k, wl.block

    def step():
        sel = ssa.ssa_select_blocks(q, k, blk, K)
        return ssa.ssa_attn_fwd(q, k, v, sel, blk, K, ssa.DUAL_ACTIVE_SPARSE, want_lse=False)

    ms = wall_ms(step, reps)
    ms_sel = wall_ms(lambda: ssa.ssa_select_blocks(q, k, blk, K), reps)
    pf, ps = pairs(wl.seqlen, blk, K)
    fl = 4.0 * wl.head_dim * (pf + ps) * wl.batch * wl.hq
    return {"workload": wl.name, "ms": round(ms, 3), "select_ms": round(ms_sel, 3),
            "fwd_TFLOP/s": round(fl / ((ms - ms_sel) / 1e3) / 1e12, 1),
            "tokens_per_s": round(wl.batch * wl.seqlen / (ms / 1e3), 1),
            "step": "select + dual forward (4 d (P_full + P_sparse) B Hq forward flops)"}


def multilayer(ssa, dev, seed, steps=10, warmup=3):
    """Four layers (B=4, 32/8 heads, N=8192, top_k 16) with their own inputs:
    per step every layer's selection and dual forward, then every layer's
    backward from the last, the active stream drawn per step and shared by
    the layers; ``steps`` timed steps after ``warmup``; tokens/s =
    steps B N / t_total."""
    import torch

    import ssa_inputs as si

    wl = si.WORKLOADS["multilayer_b4_n8k_l4"]
    K, blk = wl.top_k, wl.block
    layers = []
    for layer in range(wl.layers):
        q, k, v, _ = si.draw_qkv(wl, seed, layer, device=str(dev))
        layers.append((q, k, v, si.draw_dout(wl, seed, layer, device=str(dev))))
    modes = [ssa.DUAL_ACTIVE_FULL if m == 0 else ssa.DUAL_ACTIVE_SPARSE
             for m in si.draw_modes(seed, warmup + steps)]

    def step(mode):
        saved = []
        for q, k, v, _ in layers:
            sel = ssa.ssa_select_blocks(q, k, blk, K)
            saved.append((sel, ssa.ssa_attn_fwd(q, k, v, sel, blk, K, mode)))
        for (q, k, v, g), (sel, fwd) in zip(reversed(layers), reversed(saved)):
            ssa.ssa_attn_bwd(q, k, v, sel, fwd, g, blk, K, mode)

    for i in range(warmup):
        step(modes[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(modes[warmup + i])
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    pf, ps = pairs(wl.seqlen, blk, K)
    fl = 14.0 * wl.head_dim * (pf + ps) * wl.batch * wl.hq * wl.layers
    return {"workload": wl.name, "steps": steps, "warmup": warmup, "seconds": round(t, 4),
            "ms_per_step": round(t * 1e3 / steps, 3), "tokens_per_s": round(steps * wl.batch * wl.seqlen / t, 1),
            "TFLOP/s": round(steps * fl / t / 1e12, 2),
            "frac_of_bf16_peak": round(steps * fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def head64_layer(ssa, dev, seed, steps=10, warmup=3):
    """The training layer with 64-wide heads (B=2, 32/8 heads, N=16384, d=64,
    block 64, top_k 16: the head size of the pages' 1B model): ``steps`` timed
    training steps (selection, dual forward, backward) after ``warmup``, the
    active stream drawn per step."""
    import torch

    import ssa_inputs as si

    wl = si.scaled_down(si.WORKLOADS["train_b2_h32_n16k"], name="train_b2_h32_n16k_d64", head_dim=64)
    q, k, v, _ = si.draw_qkv(wl, seed, device=str(dev))
    dout = si.draw_dout(wl, seed, device=str(dev))
    modes = [ssa.DUAL_ACTIVE_FULL if m == 0 else ssa.DUAL_ACTIVE_SPARSE
             for m in si.draw_modes(seed, warmup + steps)]
    K, blk = wl.top_k, wl.block
    train_steps(ssa, q, k, v, dout, blk, K, modes[:warmup])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    train_steps(ssa, q, k, v, dout, blk, K, modes[warmup:])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    pf, ps = pairs(wl.seqlen, blk, K)
    fl = 14.0 * wl.head_dim * (pf + ps) * wl.batch * wl.hq
    return {"workload": wl.name, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 3),
            "TFLOP/s": round(fl / (ms / 1e3) / 1e12, 2),
            "frac_of_bf16_peak": round(fl / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(wl.batch * wl.seqlen / (ms / 1e3), 1)}


def decode_128k(ssa, dev, reps):
    """One decode step per sequence at the end of a 131072-token cache (B=4,
    16 query / 4 KV heads, d 128, block 64, top_k 32, four planted sinks):
    SPARSE_ONLY (selection against the block-mean cache + the selected
    blocks) against FULL_ONLY (every cached key).  Bytes are the unique cache
    rows a step must read: K and V of every key of each KV head (full), or
    of the union of the blocks its G query heads selected plus the block
    means (sparse)."""
    import torch

    import ssa_inputs as si

    wl = si.WORKLOADS["decode_b4_n128k_sinks"]
    q, k, v = si.draw_decode(wl, 0, device=str(dev))
    L, blk, K, d = wl.seqlen, wl.block, wl.top_k, wl.head_dim
    mu = torch.empty(wl.batch, wl.hkv, L // blk, d, dtype=torch.float32, device=dev)
    ssa.ssa_cache_block_means(k, mu, blk, 0, L // blk)
    pos = torch.full((wl.batch,), L - 1, dtype=torch.int32, device=dev)
    sp = ssa.ssa_decode(q, k, v, mu, pos, blk, K, ssa.SPARSE_ONLY)
    ssa.ssa_decode(q, k, v, None, pos, blk, K, ssa.FULL_ONLY)
    torch.cuda.synchronize()

    def gpu_ms(mode, m):
        # the library's events around its decode launches (selection, parts,
        # merge): device time, without the host's per-call overhead
        t = kernel_times(ssa, lambda: [ssa.ssa_decode(q, k, v, m, pos, blk, K, mode) for _ in range(reps)])
        return t["decode"][0] / t["decode"][1]

    ms_sp = gpu_ms(ssa.SPARSE_ONLY, mu)
    ms_fu = gpu_ms(ssa.FULL_ONLY, None)
    row = d * k.element_size() * 2                                  # one key + one value row
    sel = sp["sel"].view(wl.batch, wl.hkv, wl.group * K).cpu()
    blocks = sum(len(set(x.tolist()) - {-1}) for x in sel.view(-1, wl.group * K))
    bytes_sp = blocks * blk * row + mu.numel() * 4
    bytes_fu = wl.batch * wl.hkv * L * row
    # chunked prefill: the last 4096 prompt tokens against the same cache
    C = 4096
    g = torch.Generator(device=dev).manual_seed(21)
    qc = torch.randn(wl.batch, wl.hq, C, d, generator=g, device=dev).to(q.dtype)

    def dev_ms(fn, names):
        fn()
        t = kernel_times(ssa, lambda: [fn() for _ in range(3)])
        return sum(t[n][0] for n in names if n in t) / 3

    pf_sp = dev_ms(lambda: ssa.ssa_prefill(qc, k, v, mu, L - C, blk, K, ssa.SPARSE_ONLY),
                   ("select", "bucket", "sparse_part", "sparse_merge"))
    pf_sel = dev_ms(lambda: ssa.ssa_prefill(qc, k, v, mu, L - C, blk, K, ssa.SPARSE_ONLY), ("select",))
    pf_fu = dev_ms(lambda: ssa.ssa_prefill(qc, k, v, None, L - C, blk, K, ssa.FULL_ONLY), ("fwd_mfma",))
    prefill = {"chunk": C, "positions": f"{L - C} .. {L - 1}", "sparse_ms": round(pf_sp, 3),
               "sparse_select_ms": round(pf_sel, 3),
               "full_ms": round(pf_fu, 3), "speedup": round(pf_fu / pf_sp, 2),
               "full_TFLOPs": round(4 * d * wl.batch * wl.hq * sum(range(L - C + 1, L + 1)) / (pf_fu / 1e3) / 1e12, 1)}
    return {"workload": wl.name, "prefill": prefill, "positions": "last token of each sequence (t = 131071)",
            "sparse_ms": round(ms_sp, 4), "full_ms": round(ms_fu, 4), "speedup": round(ms_fu / ms_sp, 2),
            "sparse_GBps": round(bytes_sp / (ms_sp / 1e3) / 1e9, 1),
            "full_GBps": round(bytes_fu / (ms_fu / 1e3) / 1e9, 1),
            "sparse_bytes": bytes_sp, "full_bytes": bytes_fu,
            "tokens_per_s_sparse": round(wl.batch / (ms_sp / 1e3), 1)}


def measured_ceilings(ssa, dev):
    """The two machine probes of libssa, timed by its own event hooks: the bf16
    matrix rate the chip sustains with every SIMD busy (two waves per SIMD,
    independent chains), and the bandwidth of a plain 1 GiB device copy
    (read + written bytes / time)."""
    import torch

    blocks, iters = 2048, 4000                   # 2 workgroups of 4 waves per CU, ~6 ms
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ssa.ssa_probe_mfma(sink, blocks, 100)
    ssa.ssa_probe_copy(src, dst)

    def both():
        for _ in range(3):
            ssa.ssa_probe_mfma(sink, blocks, iters)
            ssa.ssa_probe_copy(src, dst)

    t = kernel_times(ssa, both)
    mfma_ms, n1 = t["probe_mfma"]
    copy_ms, n2 = t["probe_copy"]
    nbytes = src.numel() * 4
    # fp32 atomics on 64 hot 16 KiB tiles (2 GiB of payload), and LDS operand
    # reads (16-byte and transposing 8-byte) with two workgroups per CU
    abuf = torch.zeros(64 * 4096, dtype=torch.float32, device=dev)
    lsink = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    ssa.ssa_probe_atomic(abuf, 2048, 4)
    ssa.ssa_probe_lds(lsink, 512, 100, 0)

    def probes():
        ssa.ssa_probe_atomic(abuf, 2048, 64)
        ssa.ssa_probe_lds(lsink, 512, 20000, 0)
        ssa.ssa_probe_lds(lsink, 512, 20000, 1)

    t2 = kernel_times(ssa, probes)
    at_ms, _ = t2["probe_atomic"]
    lds_tot, _ = t2["probe_lds"]
    t3 = kernel_times(ssa, lambda: ssa.ssa_probe_lds(lsink, 512, 20000, 1))
    tr_ms = t3["probe_lds"][0]
    b128_ms = lds_tot - tr_ms
    lds_reads = 512 * 4 * 20000 * 8
    return {"mfma_bf16_tflops": round(blocks * 16 * iters * 32768 / (mfma_ms / n1 / 1e3) / 1e12, 1),
            "copy_gbs": round(2 * nbytes / (copy_ms / n2 / 1e3) / 1e9, 1),
            "atomic_f32_gbs": round(2048 * 64 * 16384 / (at_ms / 1e3) / 1e9, 1),
            "lds_read_b128_tbs": round(lds_reads * 1024 / (b128_ms / 1e3) / 1e12, 1),
            "lds_read_tr_b64_tbs": round(lds_reads * 512 / (tr_ms / 1e3) / 1e12, 1),
            "note": "dense 32x32x16 bf16 matrix loop on every SIMD; 1 GiB device copy (read + write); fp32 "
                    "global atomics on hot tiles (payload bytes); LDS reads chip-wide, 16-byte and transposing "
                    "8-byte per lane"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_library() -> str:
    try:
        import threadpoolctl

        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            return f"{i.get('internal_api', '?')} {i.get('version', '')} ({os.path.basename(i.get('filepath', ''))})"
    except Exception:                       # noqa: BLE001 -- informational only
        pass
    return "unknown"


def cpu_baseline(wl, K, seed, q, k, v, dout, mode):
    """The fp64 oracle on the host's cores: one whole (batch 0, KV head 0)
    unit of the training step -- selection, both streams and the backward of
    its G query heads over all N rows, every key of the KV head -- on a
    process pool with one BLAS thread per worker, scaled by the layer's
    B * Hkv units to seconds per step."""
    import numpy as np

    import ssa_inputs as si
    from oracle import parallel

    G, d = wl.group, wl.head_dim
    b, c = 0, 0
    hs = slice(c * G, (c + 1) * G)
    res = parallel.unit_step(si.to_f64(q[b, hs]), si.to_f64(k[b, c]), si.to_f64(v[b, c]), wl.block, K,
                             1.0 / float(np.sqrt(d)), mode, dout_u=si.to_f64(dout[b, hs]), M=q.numel())
    pf, ps = pairs(wl.seqlen, wl.block, K)
    unit_flops = 14.0 * d * (pf + ps) * G
    units = wl.batch * wl.hkv
    sec = res["seconds"]
    return {"value": unit_flops / sec / 1e12, "unit": "TFLOP/s", "cores": res["workers"], "kind": "oracle",
            "seconds_unit": round(sec, 3), "units_per_step": units, "seconds_per_step": round(sec * units, 2),
            "cpu_model": _cpu_model(), "blas": _blas_library(),
            "sample": f"one whole (batch {b}, KV head {c}) unit of {wl.name} at top_k {K}: selection, both "
                      f"streams and the backward of its {G} query heads over all {wl.seqlen} rows, every key "
                      f"of the KV head; fp64 numpy oracle on {res['workers']} worker processes (1 BLAS thread "
                      f"each); {unit_flops:.4g} algorithmic flops; scaled by the {units} units of the layer"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the attention path has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import torch

    import ssa_inputs as si

    wl = si.WORKLOADS[args.workload]
    changes = {}
    if args.seqlen:
        changes["seqlen"] = args.seqlen
    if args.batch:
        changes["batch"] = args.batch
    if changes:
        wl = si.scaled_down(wl, **changes)
    K = args.top_k or wl.top_k
    q_c, k_c, v_c, _ = si.draw_qkv(wl, args.seed)
    dout_c = si.draw_dout(wl, args.seed)
    modes_bits = si.draw_modes(args.seed, args.warmup + args.steps)

    # the CPU leg runs first, before the GPU is touched (its worker processes
    # start from a process without GPU state)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, K, args.seed, q_c, k_c, v_c, dout_c, 1 if modes_bits[0] else 0)

    import block_sparse_full_ssa_amd as ssa

    dev = torch.device("cuda:0")
    q, k, v, dout = (x.to(dev) for x in (q_c, k_c, v_c, dout_c))
    del q_c, k_c, v_c, dout_c
    modes = [ssa.DUAL_ACTIVE_FULL if m == 0 else ssa.DUAL_ACTIVE_SPARSE for m in modes_bits]
    torch.cuda.synchronize()

    B, Hq, N, d = wl.batch, wl.hq, wl.seqlen, wl.head_dim
    blk = wl.block
    # headline: W warm-up steps, then K timed steps with the event timing off
    train_steps(ssa, q, k, v, dout, blk, K, modes[:args.warmup])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    train_steps(ssa, q, k, v, dout, blk, K, modes[args.warmup:])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    # per-kernel device times: the same steps again with events on every launch
    t1 = time.perf_counter()
    kt = kernel_times(ssa, lambda: train_steps(ssa, q, k, v, dout, blk, K, modes[args.warmup:]))
    ms_events = (time.perf_counter() - t1) * 1000.0 / args.steps
    kernels = {n: {"total_ms": t, "launches": c, "avg_ms": t / c} for n, (t, c) in kt.items()}
    pf, ps = pairs(N, blk, K)
    flops = 14.0 * d * (pf + ps) * B * Hq
    tflops = flops / (ms / 1000.0) / 1e12

    # dominant kernel and its roofline
    dom = max(kernels, key=lambda n: kernels[n]["total_ms"])
    per_launch = algorithmic_flops_per_launch(d, pf, ps, B * Hq)
    roofline = None
    if dom in per_launch:
        achieved = per_launch[dom] / (kernels[dom]["avg_ms"] / 1000.0) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(dom, wl.name, K),
                    "flops_per_launch": per_launch[dom]}
    kernel_frac = {n: round(per_launch[n] / (kk["avg_ms"] / 1000.0) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                   for n, kk in kernels.items() if n in per_launch}

    sweep = None
    if not args.no_sweep and wl.top_k_sweep:
        sweep = {}
        n_sw = max(4, args.steps // 2)
        cyc = [modes[i % len(modes)] for i in range(2 + n_sw)]
        for kk in wl.top_k_sweep:
            train_steps(ssa, q, k, v, dout, blk, kk, cyc[:2])
            torch.cuda.synchronize()
            ts = time.perf_counter()
            train_steps(ssa, q, k, v, dout, blk, kk, cyc[2:])
            torch.cuda.synchronize()
            m2 = (time.perf_counter() - ts) * 1000.0 / n_sw
            a, b = pairs(N, blk, kk)
            f2 = 14.0 * d * (a + b) * B * Hq
            sweep[str(kk)] = {"ms_per_step": round(m2, 3), "TFLOP/s": round(f2 / (m2 / 1000) / 1e12, 2),
                              "frac_of_bf16_peak": round(f2 / (m2 / 1000) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "tokens_per_s": round(B * N / (m2 / 1000.0), 1)}

    single = None
    if not args.no_single_stream:
        ks = list(wl.top_k_sweep) if (not args.no_sweep and wl.top_k_sweep) else [K]
        single = single_stream(ssa, q, k, v, dout, blk, K, ks, max(3, args.steps // 2))
    del q, k, v, dout
    torch.cuda.empty_cache()

    others = {}
    if not args.no_other_layers:
        others["long_n64k_sinks"] = long_layer(ssa, dev, args.seed, 3)
        torch.cuda.empty_cache()
        others["multilayer_b4_n8k_l4"] = multilayer(ssa, dev, args.seed)
        others["train_b2_h32_n16k_d64"] = head64_layer(ssa, dev, args.seed)
        torch.cuda.empty_cache()

    decode = None if args.no_decode else decode_128k(ssa, dev, max(10, args.steps))
    ceilings = measured_ceilings(ssa, dev)
    if roofline is not None:
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / ceilings["mfma_bf16_tflops"], 4)
    if cpu is not None:
        cpu["gpu_speedup"] = round(cpu["seconds_per_step"] / (ms / 1e3), 1)

    line = {
        "metric": "SSA fwd+bwd attention TFLOP/s and tokens/s at 16K ctx; % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads_q": Hq, "heads_kv": wl.hkv, "seq_len": N,
                   "head_dim": d, "block": blk, "top_k": K,
                   "step": "select + dual fwd + bwd, active stream 50/50 per step"},
        "tokens_per_s": round(B * N / (ms / 1000.0), 1),
        "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "algorithmic_flops_per_step": flops,
        "ms_per_step_with_kernel_events": round(ms_events, 3),
        "kernels_ms_avg": {n: round(kk["avg_ms"], 4) for n, kk in kernels.items()},
        "roofline": roofline,
        "kernel_frac_of_bf16_peak": kernel_frac,
        "matrix_pipe_use": dict(matrix_pipe_use(("bwd_mfma", "fwd_mfma", "bwd_dq", "bwd_sparse"), wl.name, K),
                                source="profiles/mfma_util_train_b2_h32_n16k.md (rocprofv3 --pmc MfmaUtil)"),
        "measured_ceilings": ceilings,
        "frac_of_measured_mfma": round(tflops / ceilings["mfma_bf16_tflops"], 4),
        "cpu_baseline": cpu,
    }
    if sweep:
        line["top_k_sweep"] = sweep
    if single:
        line.update(single)
    line.update(others)
    line["decode_128k"] = decode
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
