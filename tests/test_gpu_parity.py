"""GPU parity of the HIP path against the CPU oracle (through the C interface).

Selection must match bit for bit on screened inputs (no two scores within
1e-3 at any cutoff tested); floating-point outputs within the tolerances in
gpu_cases.  Cases span several tiles, ragged tails, the block sizes 32 / 64 /
128, GQA groups 1..4, top_k = 1 and top_k >= number of blocks.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import ssa_inputs as si

from gpu_cases import (TOL, assert_close, assert_normwise, excess, inputs, oracle_fwd, oracle_select,
                       scale_of, to_dev)

pytestmark = pytest.mark.gpu

W = si.WORKLOADS
TINY = W["tiny_mha_n256_fp32"]
# bf16 layers small enough for the oracle, each spanning several 128-query tiles
SMALL = {
    "gqa_n512_b64_k4": si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=2, top_k=4),
    "gqa_n320_ragged": si.scaled_down(W["gqa_n4k_fwd"], seqlen=320, hq=4, hkv=1, top_k=3),
    "mha_n384_b32_k5": si.scaled_down(W["gqa_n4k_fwd"], seqlen=384, hq=2, hkv=2, block=32, top_k=5),
    "gqa_n512_b128_k2": si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=4, hkv=1, block=128, top_k=2),
    "sinks_n1024_k8": si.scaled_down(W["long_n64k_sinks"], seqlen=1024, hq=4, hkv=1, top_k=8),
    "gqa_n256_d64": si.scaled_down(W["gqa_n4k_fwd"], seqlen=256, hq=2, hkv=1, head_dim=64, top_k=2),
    # d = 64 on the matrix kernels: 32-key blocks with a ragged last query tile,
    # and 128-key blocks (four key halves per block in the bucket kernels)
    "gqa_n640_d64_b32_k5": si.scaled_down(W["gqa_n4k_fwd"], seqlen=640, hq=4, hkv=2, block=32, head_dim=64,
                                          top_k=5),
    "mha_n512_d64_b128_k2": si.scaled_down(W["gqa_n4k_fwd"], seqlen=512, hq=2, hkv=2, block=128, head_dim=64,
                                           top_k=2),
    # N an odd multiple of 32: the last 64-key tile of the dual forward and
    # the dQ kernel (and of the d = 64 forward) reaches past the keys, whose
    # copies read zeros that the causal mask removes
    "mha_n352_b32_k4": si.scaled_down(W["gqa_n4k_fwd"], seqlen=352, hq=2, hkv=1, block=32, top_k=4),
    "gqa_n288_d64_b32_k3": si.scaled_down(W["gqa_n4k_fwd"], seqlen=288, hq=4, hkv=2, block=32, head_dim=64,
                                          top_k=3),
}
MODES = [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE, oracle.FULL_ONLY, oracle.SPARSE_ONLY]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_full_ssa_amd  # noqa: F401  (fails loudly when libssa is missing)


def ssa():
    import block_sparse_full_ssa_amd as m
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_fwd(name, wl, out, ref, mode):
    dt = wl.dtype
    if mode != oracle.SPARSE_ONLY:
        assert_close(f"{name} h_full", out["h_full"], ref["h_full"], dt)
        assert_close(f"{name} lse_full", out["lse_full"], ref["lse_full"], dt)
    if mode != oracle.FULL_ONLY:
        assert_close(f"{name} h_sparse", out["h_sparse"], ref["h_sparse"], dt)
        assert_close(f"{name} lse_sparse", out["lse_sparse"], ref["lse_sparse"], dt)
    if mode in (oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE):
        assert_close(f"{name} delta", out["delta"], ref["delta"], dt)
        L = out["losses"].cpu().numpy()
        rtol = TOL[dt][1]
        assert L[0] == L[1]
        assert abs(L[0] - ref["L_sparsity"]) <= rtol * ref["L_sparsity"] + 1e-30, (L, ref["L_sparsity"])


# ------------------------------------------------------------------ select --

@pytest.mark.parametrize("name", ["tiny"] + list(SMALL))
def test_select_matches_oracle(name):
    wl = TINY if name == "tiny" else SMALL[name]
    _say(f"select {name}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd = to_dev(q, k)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    want, _ = oracle_select(wl, 0, (wl.top_k,), wl.top_k)
    assert np.array_equal(sel.cpu().numpy(), want)


def test_select_topk_sweep_gqa_n2048():
    """top_k 4, 8, 16, 32 of the 16K training layer's sweep, on a 2048-token slice."""
    wl = si.scaled_down(W["train_b2_h32_n16k"], batch=1, seqlen=2048, hq=4, hkv=1)
    ks = (4, 8, 16, 32)
    (q, k, v), _ = inputs(wl, 0, ks)
    qd, kd = to_dev(q, k)
    for K in ks:
        _say(f"select sweep K={K}")
        sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
        want, _ = oracle_select(wl, 0, ks, K)
        assert np.array_equal(sel.cpu().numpy(), want), K


def test_select_all_blocks_and_top1():
    wl = SMALL["gqa_n512_b64_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd = to_dev(q, k)
    for K in (1, 8, 11, 100):            # nb = 8: 8, 11 and 100 select everything
        sel = ssa().ssa_select_blocks(qd, kd, wl.block, K).cpu().numpy()
        want, _ = oracle_select(wl, 0, (wl.top_k,), K)
        assert np.array_equal(sel, want), K


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_select_chunked_candidates_all_rows(dtype):
    """530 key blocks: candidates are scored and ranked in chunks of 256 with
    each row's winners carried between chunks (256 + 256 + a ragged 18).
    Every row bit for bit, top_k 8 and 64 (63 carried winners, the most), on
    a bf16 layer (two-term bf16 scores) and an fp32 one (fp32 scores)."""
    wl = si.scaled_down(W["gqa_n4k_fwd"], seqlen=32 * 530, hq=2, hkv=1, block=32, head_dim=64, top_k=8,
                        dtype=dtype)
    ks = (8, 64)
    (q, k, v), _ = inputs(wl, 0, ks)
    qd, kd = to_dev(q, k)
    for K in ks:
        _say(f"select chunked nb 530 {dtype} K={K}")
        sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
        want, _ = oracle_select(wl, 0, ks, K)
        assert np.array_equal(sel.cpu().numpy(), want), K


# ----------------------------------------------------------------- forward --

@pytest.mark.parametrize("mode", MODES)
def test_fwd_tiny_fp32(mode):
    wl = TINY
    _say(f"fwd tiny mode {mode}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = torch.from_numpy(oracle_select(wl, 0, (wl.top_k,), wl.top_k)[0]).to("cuda:0")
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode)
    torch.cuda.synchronize()
    _check_fwd("tiny", wl, out, oracle_fwd(wl, 0, (wl.top_k,), wl.top_k, mode), mode)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.FULL_ONLY, oracle.SPARSE_ONLY])
@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_small_bf16(name, mode):
    wl = SMALL[name]
    _say(f"fwd {name} mode {mode}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = torch.from_numpy(oracle_select(wl, 0, (wl.top_k,), wl.top_k)[0]).to("cuda:0")
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode)
    torch.cuda.synchronize()
    _check_fwd(name, wl, out, oracle_fwd(wl, 0, (wl.top_k,), wl.top_k, mode), mode)


@pytest.mark.parametrize("mode", [oracle.FULL_ONLY, oracle.DUAL_ACTIVE_FULL])
@pytest.mark.parametrize("name", ["gqa_n512_b64_k4", "gqa_n256_d64"])
def test_fwd_late_logit_spike(name, mode):
    """Queries 200.. of one head meet at key 200 a logit about 100 (log2
    units) above every earlier logit of theirs, so the reference maximum of
    their softmax has to move mid-row by more than 2^64 (the full stream
    alone moves it only when a tile's weights would exceed 2^64); every output
    still matches the oracle."""
    wl = SMALL[name]
    _say(f"fwd late logit spike {name} mode {mode}")
    (q, k, v), _ = inputs(wl, 0, ())
    q, k = q.clone(), k.clone()               # the cached inputs of the other tests stay as drawn
    u = torch.zeros(wl.head_dim)
    u[0] = 1.0
    t0 = 200
    q[0, 0, t0:] = u.to(q.dtype)              # query head 0 reads KV head 0
    k[0, 0, t0] = (800.0 * u).to(k.dtype)     # logit 800 / sqrt(d) > 70 nats
    qf, kf, vf = (si.to_f64(x) for x in (q, k, v))
    sel, _ = oracle.select_blocks(qf, kf, wl.block, wl.top_k, wl.group)
    qd, kd, vd = to_dev(q, k, v)
    out = ssa().ssa_attn_fwd(qd, kd, vd, torch.from_numpy(sel).to("cuda:0"), wl.block, wl.top_k, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(qf, kf, vf, sel, wl.block, scale_of(wl), wl.group, mode)
    assert float(ref["lse_full"][0, 0, t0:].min()) > 64 * math.log(2.0)    # the spike dominates
    _check_fwd(f"spike {name}", wl, out, ref, mode)


@pytest.mark.parametrize("top_k", [1, 2, 8, 11])
def test_sparse_only_fwd_topk_extremes(top_k):
    """SPARSE_ONLY on key-block buckets when each query keeps only its own
    block (top_k 1, every bucket holds just its own block's rows), one
    earlier block, or every block (top_k = N / block and above)."""
    wl = SMALL["gqa_n512_b64_k4"]
    ks = (top_k,) if top_k == 2 else ()
    _say(f"sparse-only fwd top_k {top_k}")
    (q, k, v), _ = inputs(wl, 0, ks)
    qd, kd, vd = to_dev(q, k, v)
    sel = torch.from_numpy(oracle_select(wl, 0, ks, top_k)[0]).to("cuda:0")
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, top_k, oracle.SPARSE_ONLY)
    torch.cuda.synchronize()
    ref = oracle_fwd(wl, 0, ks, top_k, oracle.SPARSE_ONLY)
    _check_fwd(f"top_k {top_k}", wl, out, ref, oracle.SPARSE_ONLY)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_SPARSE, oracle.FULL_ONLY, oracle.SPARSE_ONLY])
def test_fwd_gqa_n4k_full_layer(mode):
    """The 4K GQA layer (16 query / 4 KV heads, d 128, block 64, top_k 16) whole.

    Its late query tiles contain waves for which no row selects some key
    tile, which exercises the skip of the sparse update (a wave-uniform
    branch around matrix instructions).
    """
    wl = W["gqa_n4k_fwd"]
    _say(f"fwd gqa_n4k_fwd full layer mode {mode}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    want_sel, _ = oracle_select(wl, 0, (wl.top_k,), wl.top_k)
    assert np.array_equal(sel.cpu().numpy(), want_sel)
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode)
    torch.cuda.synchronize()
    ref_mode = oracle.DUAL_ACTIVE_FULL if mode == oracle.DUAL_ACTIVE_SPARSE else mode
    _check_fwd("gqa_n4k", wl, out, oracle_fwd(wl, 0, (wl.top_k,), wl.top_k, ref_mode), ref_mode)


@pytest.mark.parametrize("name", ["tiny", "gqa_n512_b64_k4", "mha_n384_b32_k5"])
def test_all_blocks_selected_streams_identical(name):
    """top_k >= number of blocks: h_sparse == h_full bit for bit and delta == 0."""
    wl = TINY if name == "tiny" else SMALL[name]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    K = wl.nblocks + 1
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, K, oracle.DUAL_ACTIVE_FULL)
    torch.cuda.synchronize()
    assert torch.equal(out["h_full"], out["h_sparse"])
    assert torch.equal(out["lse_full"], out["lse_sparse"])
    assert float(out["delta"].abs().max()) == 0.0
    assert float(out["losses"][0]) == 0.0


@pytest.mark.parametrize("name", ["tiny", "sinks_n1024_k8"])
def test_delta_bound_on_gpu_outputs(name):
    """||h_full - h_sparse|| <= 2 delta max||v|| per query (up to output rounding)."""
    wl = TINY if name == "tiny" else SMALL[name]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.DUAL_ACTIVE_FULL)
    torch.cuda.synchronize()
    diff = (out["h_full"].double() - out["h_sparse"].double()).norm(dim=-1).cpu()
    vmax = v.double().norm(dim=-1).max()
    slack = 1e-5 if wl.dtype == torch.float32 else 2 ** -7 * float(out["h_full"].double().norm(dim=-1).max())
    assert bool((diff <= 2 * out["delta"].double().cpu() * vmax + slack).all())


def test_fwd_deterministic():
    wl = SMALL["gqa_n512_b64_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    a = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.DUAL_ACTIVE_FULL)
    b = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.DUAL_ACTIVE_FULL)
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta", "losses"):
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------ diagnostics --

# Statistics are fp32 outputs computed from the same rounded inputs as the
# oracle; their error is the fp32 rounding of the logits (|z| <~ 30, ~1e-6)
# and of ln2 (log2 l - A / l) with log2 l <~ 20 (~1e-5).
STATS_TOL = {torch.bfloat16: (1e-4, 1e-4), torch.float32: (1e-5, 1e-5)}


@functools.lru_cache(maxsize=None)
def _oracle_stats(name):
    wl = TINY if name == "tiny" else SMALL[name]
    _, (qf, kf, _) = inputs(wl, 0, (wl.top_k,))
    return oracle.full_stats(qf, kf, wl.block, scale_of(wl), wl.group)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.FULL_ONLY])
@pytest.mark.parametrize("name", ["tiny"] + list(SMALL))
def test_fwd_stats_match_oracle(name, mode):
    """Sink-block mass, entropy and their per-head means against the oracle;
    the attention outputs of the statistics pass equal those of the plain
    forward bit for bit."""
    wl = TINY if name == "tiny" else SMALL[name]
    _say(f"fwd stats {name} mode {mode}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = torch.from_numpy(oracle_select(wl, 0, (wl.top_k,), wl.top_k)[0]).to("cuda:0")
    out = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode, stats=True)
    plain = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode)
    torch.cuda.synchronize()
    sink, ent, means = _oracle_stats(name)
    atol, rtol = STATS_TOL[wl.dtype]
    for key, got, want in (("sink_mass", out["sink_mass"], sink), ("entropy", out["entropy"], ent),
                           ("head_stats", out["head_stats"], means)):
        e = excess(got, want, atol, rtol)
        assert e <= 0, f"{name} {key}: exceeds tolerance by {e:.3g}"
    for key in ("h_full", "lse_full", "h_sparse", "lse_sparse", "delta", "losses"):
        if key in plain:
            assert torch.equal(out[key], plain[key]), key


def test_fwd_stats_sparse_only_unsupported():
    wl = SMALL["gqa_n512_b64_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    with pytest.raises(ssa().SSAError):
        ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.SPARSE_ONLY, stats=True)


# ---------------------------------------------------------------- backward --

def _bwd_case(wl, mode, with_dout=True, ws=0.7, wc=1.3):
    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    g = si.draw_dout(wl, 0)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    osel = oracle_select(wl, 0, (wl.top_k,), wl.top_k)[0]
    sel = torch.from_numpy(osel).to("cuda:0")
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, mode)
    dq, dk, dv = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd if with_dout else None, wl.block,
                                    wl.top_k, mode, ws, wc)
    torch.cuda.synchronize()
    ref_f = oracle_fwd(wl, 0, (wl.top_k,), wl.top_k, mode)
    rq, rk, rv = oracle.backward(qf, kf, vf, None if mode == oracle.FULL_ONLY else osel, wl.block,
                                 scale_of(wl), wl.group, mode, si.to_f64(g) if with_dout else None,
                                 ws, wc, fwd=ref_f)
    return (dq, dk, dv), (rq, rk, rv)


@pytest.mark.parametrize("mode", MODES)
def test_bwd_tiny_fp32(mode):
    _say(f"bwd tiny mode {mode}")
    got, want = _bwd_case(TINY, mode)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_close(f"tiny {n}", a, b, torch.float32)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE])
def test_bwd_tiny_alignment_only(mode):
    """No upstream gradient: only L_sparsity / L_commit move q, k, v."""
    _say(f"bwd tiny alignment-only mode {mode}")
    got, want = _bwd_case(TINY, mode, with_dout=False, ws=1.0, wc=1.0)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_normwise(f"tiny align {n}", a, b, 1e-4)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["gqa_n512_b64_k4", "gqa_n320_ragged", "mha_n384_b32_k5",
                                  "gqa_n512_b128_k2", "gqa_n256_d64"])
def test_bwd_small_bf16(name, mode):
    _say(f"bwd {name} mode {mode}")
    got, want = _bwd_case(SMALL[name], mode)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_close(f"{name} {n}", a, b, torch.bfloat16)


@pytest.mark.parametrize("mode", [oracle.DUAL_ACTIVE_FULL, oracle.DUAL_ACTIVE_SPARSE])
def test_bwd_bf16_alignment_only(mode):
    _say(f"bwd bf16 alignment-only mode {mode}")
    got, want = _bwd_case(SMALL["gqa_n512_b64_k4"], mode, with_dout=False, ws=1.0, wc=1.0)
    for n, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_normwise(f"bf16 align {n}", a, b, 1e-2)


def test_sparse_only_gradient_deficiency():
    """SPARSE_ONLY: a key outside every query's support gets dk = dv = 0 exactly.

    With the upstream gradient on a single query row, keys of blocks that row
    did not select receive nothing from the sparse stream.
    """
    wl = SMALL["gqa_n512_b64_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = to_dev(q, k, v)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    g = torch.zeros_like(qd)
    t = 500
    g[0, 0, t] = 1.0
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.SPARSE_ONLY)
    dq, dk, dv = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, g, wl.block, wl.top_k, oracle.SPARSE_ONLY)
    torch.cuda.synchronize()
    chosen = set(int(x) for x in sel[0, 0, t].cpu() if x >= 0)
    outside = [i for i in range(t + 1) if i // wl.block not in chosen]
    assert len(outside) > 0
    assert float(dk[0, 0, outside].abs().max()) == 0.0
    assert float(dv[0, 0, outside].abs().max()) == 0.0
    inside = [i for i in range(t + 1) if i // wl.block in chosen]
    assert float(dv[0, 0, inside].abs().max()) > 0.0


# --------------------------------------------------- ignored sel entries --

def _spliced_sel(sel: torch.Tensor, block: int, nb: int) -> torch.Tensor:
    """sel with the first -1 slot of each padded row replaced by an entry the
    kernels must ignore: a repeat of the entry before it (rows t % 3 == 0), a
    block above the row's own one (t % 3 == 1: own + 1 when it exists, else
    nb), or a block far past the last (t % 3 == 2: 2^20, beyond any row's
    selection words).  Non-negative entries stay ascending."""
    s = sel.cpu().clone()
    B, H, N, K = s.shape
    t = torch.arange(N)
    own = t // block
    for b in range(B):
        for h in range(H):
            rows = s[b, h]
            pad = (rows < 0).int().argmax(dim=1)           # first -1 slot
            has_pad = (rows < 0).any(dim=1)
            for r in torch.nonzero(has_pad).flatten().tolist():
                p = int(pad[r])
                kind = r % 3
                if kind == 0:
                    val = int(rows[r, p - 1])
                elif kind == 1:
                    val = int(own[r]) + 1 if int(own[r]) + 1 < nb else nb
                else:
                    val = 1 << 20
                rows[r, p] = val
    return s.to(sel.device)


@pytest.mark.parametrize("mode", MODES[:2] + [oracle.SPARSE_ONLY])
@pytest.mark.parametrize("name", ["tiny", "gqa_n512_b64_k4", "mha_n384_b32_k5"])
def test_ignored_sel_entries_bit_identical(name, mode):
    """Entries naming no causal block (above the own block, past the last
    block) and repeated entries change nothing: forward and backward outputs
    equal those of the clean selection bit for bit."""
    wl = TINY if name == "tiny" else SMALL[name]
    K = wl.top_k + 2                                   # every early row is padded
    _say(f"ignored sel entries {name} mode {mode}")
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    g = si.draw_dout(wl, 0)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, K)
    bad = _spliced_sel(sel, wl.block, wl.nblocks)
    assert not torch.equal(bad, sel)
    outs = []
    for s in (sel, bad):
        fwd = ssa().ssa_attn_fwd(qd, kd, vd, s, wl.block, K, mode)
        grads = ssa().ssa_attn_bwd(qd, kd, vd, s, fwd, gd, wl.block, K, mode)
        outs.append((fwd, grads))
    torch.cuda.synchronize()
    (fa, ga), (fb, gb) = outs
    for key in ("h_full", "h_sparse", "lse_full", "lse_sparse", "delta", "losses"):
        if key in fa:
            assert torch.equal(fa[key], fb[key]), key
    for n, a, b in zip(("dq", "dk", "dv"), ga, gb):
        # the generic (fp32) path adds dk / dv with fp32 atomics, which may
        # add in another order: those compare within the dtype's tolerance
        if wl.dtype == torch.bfloat16:
            assert torch.equal(a, b), n
        else:
            assert_close(n, a, b.double().cpu().numpy(), wl.dtype)


def test_sparse_only_backward_deterministic():
    """SPARSE_ONLY backward twice on the same inputs: dq, dk, dv bit for bit
    (dq is merged from per-block partials in selection order, no atomics)."""
    wl = SMALL["gqa_n512_b64_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    g = si.draw_dout(wl, 0)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    fwd = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, oracle.SPARSE_ONLY)
    a = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, wl.top_k, oracle.SPARSE_ONLY)
    b = ssa().ssa_attn_bwd(qd, kd, vd, sel, fwd, gd, wl.block, wl.top_k, oracle.SPARSE_ONLY)
    torch.cuda.synchronize()
    for n, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), n
