"""Throughput of one SSA training step of attention on one MI355X.

A step is the whole hot path over one batch of the 16K-context training
layer (B=2, 32 query / 8 KV heads, N=16384, d=128, bf16, block 64, top_k 16
by default): block selection, the dual-stream forward (full and sparse
outputs, delta, alignment losses) and the backward with the active stream
drawn 50/50 per step from the seed.  Inputs are synthetic and resident in
HBM before timing starts.

Reported (one JSON line): algorithmic TFLOP/s of the step, tokens/s, the
roofline of the dominant kernel (its algorithmic flops per launch over its
HIP-event-timed average launch), the CPU oracle timed on a bounded sample of
the same workload, the FULL_ONLY fwd+bwd rate on the same layer and the
sparse-stream forward speedup t(FULL_ONLY fwd) / t(SPARSE_ONLY fwd).

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


def measured_traffic(kernel, workload, top_k):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated by a plain copy), or None when
    there is none for this workload or the kernel's source changed since."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
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
    return rec["bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train_b2_h32_n16k")
    ap.add_argument("--top-k", type=int, default=None)
    ap.add_argument("--seqlen", type=int, default=None, help="override N (experiments only)")
    ap.add_argument("--batch", type=int, default=None, help="override B (experiments only)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sweep", action="store_true", help="also time every top_k of the workload's sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the 128K-cache decode leg")
    ap.add_argument("--no-single-stream", action="store_true",
                    help="skip the FULL_ONLY / SPARSE_ONLY measurements")
    ap.add_argument("--cpu-rows", type=int, default=12288, help="query rows in the CPU-oracle sample")
    return ap.parse_args()


def run_steps(ssa, q, k, v, dout, wl, K, modes, steps, warmup):
    import torch

    def step(mode):
        sel = ssa.ssa_select_blocks(q, k, wl.block, K)
        fwd = ssa.ssa_attn_fwd(q, k, v, sel, wl.block, K, mode)
        grads = ssa.ssa_attn_bwd(q, k, v, sel, fwd, dout, wl.block, K, mode)
        return fwd, grads

    for i in range(warmup):
        step(modes[i])
    torch.cuda.synchronize()
    ssa.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        out = step(modes[warmup + i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernels = {}
    for name in ssa.kernel_names():
        ms, n = ssa.timing_query(name)
        if n:
            kernels[name] = {"total_ms": ms, "launches": n, "avg_ms": ms / n}
    ssa.timing_enable(False)
    del out
    return (t1 - t0) * 1000.0 / steps, kernels


def time_calls(fn, reps, warm=1):
    """Wall-clock milliseconds per call of ``fn`` (GPU work included), after warm-up."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / reps


def hbm_rates(ssa, q, k, v, sel, wl, K, reps):
    """GB/s of the HBM-bound steps (a2 selection, a8 sparse-only forward)
    from the library's device-time events, against the 8 TB/s peak.  Bytes
    are those each step must move: selection reads q and k, writes and reads
    the block means and writes sel; the sparse-only forward reads k, v and
    sel, gathers the query row of every selected (row, block) pair into its
    key block's bucket (d bf16 values per pair), writes and reads one partial
    per pair (d bf16 values + an fp32 log-sum-exp), and writes h_sparse and
    lse_sparse."""
    B, Hq, N, d = q.shape
    blk, nb = wl.block, N // wl.block
    el = q.element_size()

    def dev_ms(fn, names):
        ssa.timing_enable(True)
        for _ in range(reps):
            fn()
        ms = sum(ssa.timing_query(n)[0] for n in names) / reps
        ssa.timing_enable(False)
        return ms

    ms_sel = dev_ms(lambda: ssa.ssa_select_blocks(q, k, blk, K), ("block_mean", "select"))
    ms_sp = dev_ms(lambda: ssa.ssa_attn_fwd(q, k, v, sel, blk, K, ssa.SPARSE_ONLY, want_lse=True),
                   ("bucket", "sparse_part", "sparse_merge"))
    mu_bytes = B * wl.hkv * nb * d * 4
    sel_bytes = q.numel() // d * K * 4
    b_sel = q.numel() * el + k.numel() * el + 2 * mu_bytes + sel_bytes
    entries = B * Hq * sum(min(K, t // blk + 1) for t in range(N))
    b_sp = (k.numel() + v.numel()) * el + sel_bytes + entries * d * el + q.numel() * el + q.numel() // d * 4 \
        + 2 * entries * (d * 2 + 4)
    return {"select_ms": round(ms_sel, 4), "select_GBps": round(b_sel / (ms_sel / 1e3) / 1e9, 1),
            "select_frac_of_hbm": round(b_sel / (ms_sel / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "sparse_fwd_ms": round(ms_sp, 4), "sparse_fwd_GBps": round(b_sp / (ms_sp / 1e3) / 1e9, 1),
            "sparse_fwd_frac_of_hbm": round(b_sp / (ms_sp / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "select_bytes": b_sel, "sparse_fwd_bytes": b_sp}


def single_stream(ssa, q, k, v, dout, wl, ks, reps):
    """FULL_ONLY fwd+bwd TFLOP/s (14 d P_full B Hq per step) and, per top_k,
    the sparse-stream forward speedup t(FULL_ONLY fwd) / t(SPARSE_ONLY fwd)
    next to P_full / P_sparse and N / (top_k block)."""
    B, Hq, N, d = q.shape
    blk = wl.block
    pf, _ = pairs(N, blk, wl.top_k)

    def full_step():
        f = ssa.ssa_attn_fwd(q, k, v, None, blk, wl.top_k, ssa.FULL_ONLY)
        ssa.ssa_attn_bwd(q, k, v, None, f, dout, blk, wl.top_k, ssa.FULL_ONLY)

    ms_full = time_calls(full_step, reps)
    ms_full_fwd = time_calls(lambda: ssa.ssa_attn_fwd(q, k, v, None, blk, wl.top_k, ssa.FULL_ONLY), reps)
    fl = 14.0 * d * pf * B * Hq
    out = {"full_only": {"ms_per_step": round(ms_full, 3), "TFLOP/s": round(fl / (ms_full / 1e3) / 1e12, 2),
                         "frac_of_bf16_peak": round(fl / (ms_full / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "fwd_ms": round(ms_full_fwd, 3),
                         "step": "FULL_ONLY fwd + bwd, 14 d P_full B Hq flops"}}
    sp = {}
    for kk in ks:
        sel = ssa.ssa_select_blocks(q, k, blk, kk)
        ms_sel = time_calls(lambda: ssa.ssa_select_blocks(q, k, blk, kk), reps)
        ms_sp = time_calls(lambda: ssa.ssa_attn_fwd(q, k, v, sel, blk, kk, ssa.SPARSE_ONLY), reps)
        a, b = pairs(N, blk, kk)
        sp[str(kk)] = {"sparse_only_fwd_ms": round(ms_sp, 3), "select_ms": round(ms_sel, 3),
                       "speedup": round(ms_full_fwd / ms_sp, 2),
                       "speedup_incl_select": round(ms_full_fwd / (ms_sp + ms_sel), 2),
                       "P_full/P_sparse": round(a / b, 2), "N/(K*block)": round(N / (kk * blk), 2),
                       "hbm": hbm_rates(ssa, q, k, v, sel, wl, kk, reps)}
        del sel
    out["sparse_fwd_speedup"] = sp

    # full-stream diagnostics (sink-block mass, entropy, per-head means) in the
    # forward pass: cost over the plain FULL_ONLY forward, and the head means
    ms_stats = time_calls(lambda: ssa.ssa_attn_fwd(q, k, v, None, blk, wl.top_k, ssa.FULL_ONLY, stats=True),
                          reps)
    st = ssa.ssa_attn_fwd(q, k, v, None, blk, wl.top_k, ssa.FULL_ONLY, stats=True)["head_stats"]
    out["full_stats"] = {"fwd_ms": round(ms_stats, 3), "overhead": round(ms_stats / ms_full_fwd - 1.0, 4),
                         "mean_sink_mass": round(float(st[..., 0].mean()), 5),
                         "mean_entropy_nats": round(float(st[..., 1].mean()), 4)}
    return out


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
    q, k, v = (x.to(dev) for x in si.draw_decode(wl, 0))
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
        ssa.timing_enable(True)
        for _ in range(reps):
            ssa.ssa_decode(q, k, v, m, pos, blk, K, mode)
        total, n = ssa.timing_query("decode")
        ssa.timing_enable(False)
        return total / n

    ms_sp = gpu_ms(ssa.SPARSE_ONLY, mu)
    ms_fu = gpu_ms(ssa.FULL_ONLY, None)
    row = d * k.element_size() * 2                                  # one key + one value row
    sel = sp["sel"].view(wl.batch, wl.hkv, wl.group * K).cpu()
    blocks = sum(len(set(x.tolist()) - {-1}) for x in sel.view(-1, wl.group * K))
    bytes_sp = blocks * blk * row + mu.numel() * 4
    bytes_fu = wl.batch * wl.hkv * L * row
    # chunked prefill: the last 4096 prompt tokens against the same cache
    C = 4096
    g = torch.Generator().manual_seed(21)
    qc = torch.randn(wl.batch, wl.hq, C, d, generator=g).to(q.dtype).to(dev)

    def dev_ms(fn, names):
        fn()
        torch.cuda.synchronize()
        ssa.timing_enable(True)
        for _ in range(3):
            fn()
        ms = sum(ssa.timing_query(n)[0] for n in names) / 3
        ssa.timing_enable(False)
        return ms

    pf_sp = dev_ms(lambda: ssa.ssa_prefill(qc, k, v, mu, L - C, blk, K, ssa.SPARSE_ONLY),
                   ("select", "bucket", "sparse_part", "sparse_merge"))
    pf_fu = dev_ms(lambda: ssa.ssa_prefill(qc, k, v, None, L - C, blk, K, ssa.FULL_ONLY), ("fwd_mfma",))
    prefill = {"chunk": C, "positions": f"{L - C} .. {L - 1}", "sparse_ms": round(pf_sp, 3),
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
    torch.cuda.synchronize()
    ssa.timing_enable(True)
    for _ in range(3):
        ssa.ssa_probe_mfma(sink, blocks, iters)
        ssa.ssa_probe_copy(src, dst)
    mfma_ms, n1 = ssa.timing_query("probe_mfma")
    copy_ms, n2 = ssa.timing_query("probe_copy")
    ssa.timing_enable(False)
    nbytes = src.numel() * 4
    return {"mfma_bf16_tflops": round(blocks * 16 * iters * 32768 / (mfma_ms / n1 / 1e3) / 1e12, 1),
            "copy_gbs": round(2 * nbytes / (copy_ms / n2 / 1e3) / 1e9, 1),
            "note": "dense 32x32x16 bf16 matrix loop on every SIMD; 1 GiB device copy (read + write)"}


def cpu_baseline(wl, K, seed, rows):
    """The fp64 oracle on the host: select + forward + backward of the last
    ``rows`` query rows of batch 0 / query head 0 (each with all its causal
    keys), as algorithmic TFLOP/s of that sample."""
    import numpy as np
    import threadpoolctl

    import oracle
    import ssa_inputs as si

    q, k, v, _ = si.draw_qkv(wl, seed)
    dout = si.draw_dout(wl, seed)
    N, d, G = wl.seqlen, wl.head_dim, wl.group
    t_idx = np.arange(N - rows, N)
    # only the KV head of query head 0 and the sampled rows are converted
    qf = si.to_f64(q[:1, :1])
    kf, vf = si.to_f64(k[:1, :1]), si.to_f64(v[:1, :1])
    gf = si.to_f64(dout[:1, :1])
    scale = 1.0 / np.sqrt(d)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    mu = oracle.block_means(kf, wl.block)
    sel_rows, _ = oracle.select_rows(qf[0, 0, t_idx], t_idx, mu[0, 0], wl.block, K)
    sel = np.full((1, 1, N, K), -1, np.int32)
    sel[0, 0, t_idx] = sel_rows
    oracle.attend_rows(qf[0, 0, t_idx], t_idx, kf[0, 0], vf[0, 0], sel_rows, wl.block, scale)
    oracle.dq_rows(qf, kf, vf, sel, wl.block, scale, 1, oracle.DUAL_ACTIVE_FULL, gf, 0, 0, t_idx)
    dt = time.perf_counter() - t0
    n_sparse = sum(min(K, t // wl.block + 1) * wl.block - (wl.block - 1 - t % wl.block) for t in t_idx)
    n_full = int((t_idx + 1).sum())
    flops = 14.0 * d * (n_full + n_sparse)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"batch 0, query head 0, last {rows} query rows with all their causal keys: "
                      f"selection + dual forward + backward (dq and these rows' dk/dv terms), fp64 numpy; "
                      f"{flops:.3g} algorithmic flops"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the attention path has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_full_ssa_amd as ssa
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
    dev = torch.device("cuda:0")
    q, k, v, _ = si.draw_qkv(wl, args.seed)
    dout = si.draw_dout(wl, args.seed)
    q, k, v, dout = (x.to(dev) for x in (q, k, v, dout))
    modes = si.draw_modes(args.seed, args.warmup + args.steps)
    modes = [ssa.DUAL_ACTIVE_FULL if m == 0 else ssa.DUAL_ACTIVE_SPARSE for m in modes]
    torch.cuda.synchronize()

    B, Hq, N, d = wl.batch, wl.hq, wl.seqlen, wl.head_dim
    ms, kernels = run_steps(ssa, q, k, v, dout, wl, K, modes, args.steps, args.warmup)
    pf, ps = pairs(N, wl.block, K)
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
    if args.sweep and wl.top_k_sweep:
        sweep = {}
        for kk in wl.top_k_sweep:
            m2, _ = run_steps(ssa, q, k, v, dout, wl, kk, modes, max(3, args.steps // 2), 1)
            a, b = pairs(N, wl.block, kk)
            sweep[str(kk)] = {"ms_per_step": round(m2, 3),
                              "TFLOP/s": round(14.0 * d * (a + b) * B * Hq / (m2 / 1000) / 1e12, 2)}

    single = None
    if not args.no_single_stream:
        ks = list(wl.top_k_sweep) if (args.sweep and wl.top_k_sweep) else [K]
        single = single_stream(ssa, q, k, v, dout, wl, ks, max(3, args.steps // 2))

    decode = None if args.no_decode else decode_128k(ssa, dev, max(10, args.steps))
    ceilings = measured_ceilings(ssa, dev)
    if roofline is not None:
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / ceilings["mfma_bf16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, K, args.seed, min(args.cpu_rows, N))

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
                   "head_dim": d, "block": wl.block, "top_k": K,
                   "step": "select + dual fwd + bwd, active stream 50/50 per step"},
        "tokens_per_s": round(B * N / (ms / 1000.0), 1),
        "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "algorithmic_flops_per_step": flops,
        "kernels_ms_avg": {n: round(kk["avg_ms"], 4) for n, kk in kernels.items()},
        "roofline": roofline,
        "kernel_frac_of_bf16_peak": kernel_frac,
        "measured_ceilings": ceilings,
        "decode_128k": decode,
        "frac_of_measured_mfma": round(tflops / ceilings["mfma_bf16_tflops"], 4),
        "cpu_baseline": cpu,
    }
    if single:
        line.update(single)
    if sweep:
        line["top_k_sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
