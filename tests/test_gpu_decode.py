"""GPU parity of single-token decode over a KV cache (through the C ABI).

A decode step for the token at position t is row t of a layer: the oracle's
selection of that row (against the block means of the cache) and both
streams of that row are the reference.  Small layers use screened inputs
(no two block scores within 1e-3 at a cutoff), so the selection must match
bit for bit; at the 128K cache the sampled heads follow the full-size rule
(rows whose fp64 margin is below 1e-3 need only a valid near-optimal
selection).  The block-mean cache is checked against the oracle's means,
including a partial update that must leave other blocks untouched.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import ssa_inputs as si
from gpu_cases import TOL, assert_close, check_selection, inputs, scale_of

pytestmark = pytest.mark.gpu

W = si.WORKLOADS
# screened layers (B = 2, so the two sequences decode at different positions)
CASES = {
    "gqa_b2_n1024_k4": si.scaled_down(W["gqa_n4k_fwd"], batch=2, seqlen=1024, hq=4, hkv=2, top_k=4),
    "mha_b2_n512_b32_k6": si.scaled_down(W["gqa_n4k_fwd"], batch=2, seqlen=512, hq=2, hkv=2, block=32, top_k=6),
    "gqa_b2_n768_b128_k3": si.scaled_down(W["gqa_n4k_fwd"], batch=2, seqlen=768, hq=4, hkv=1, block=128, top_k=3),
    "fp32_b2_n256_d64": si.scaled_down(W["tiny_mha_n256_fp32"], batch=2),
    "gqa_b2_n1024_d64_k4": si.scaled_down(W["gqa_n4k_fwd"], batch=2, seqlen=1024, hq=4, hkv=2, head_dim=64, top_k=4),
}


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


def _means(kd, block):
    B, Hkv, L, d = kd.shape
    mu = torch.full((B, Hkv, L // block, d), float("nan"), dtype=torch.float32, device=kd.device)
    ssa().ssa_cache_block_means(kd, mu, block, 0, L // block)
    return mu


@pytest.mark.parametrize("name", list(CASES))
def test_cache_block_means(name):
    wl = CASES[name]
    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    kd = k.to("cuda:0")
    mu = _means(kd, wl.block)
    torch.cuda.synchronize()
    ref = oracle.block_means(kf, wl.block)
    err = np.abs(mu.double().cpu().numpy() - ref)
    assert float(err.max()) <= 1e-6 * (1 + float(np.abs(ref).max())), float(err.max())
    # a partial update writes exactly blocks [2, 5)
    part = torch.full_like(mu, -7.0)
    ssa().ssa_cache_block_means(kd, part, wl.block, 2, 5)
    torch.cuda.synchronize()
    assert torch.equal(part[:, :, 2:5], mu[:, :, 2:5])
    assert bool((part[:, :, :2] == -7.0).all()) and bool((part[:, :, 5:] == -7.0).all())


def _positions(wl, rng):
    N, blk, K = wl.seqlen, wl.block, wl.top_k
    fixed = [0, 1, blk - 1, blk, (K - 1) * blk, K * blk - 1, K * blk, N // 2 + 3, N - blk, N - 1]
    extra = list(rng.integers(0, N, size=6))
    return sorted(set(int(x) for x in fixed + extra if 0 <= x < N))


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_layer_rows(name):
    """Both streams of decode steps at many positions (the two sequences at
    different ones) against the oracle's selection and attention of that row."""
    wl = CASES[name]
    _say(f"decode {name}")
    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    mu = _means(kd, wl.block)
    mu_ref = oracle.block_means(kf, wl.block)
    scale = scale_of(wl)
    rng = np.random.default_rng(4)
    ts = _positions(wl, rng)
    for i, t0 in enumerate(ts):
        t1 = ts[-1 - i]                                # sequence 1 decodes elsewhere
        pos = torch.tensor([t0, t1], dtype=torch.int32, device="cuda:0")
        qrow = torch.stack([qd[0, :, t0], qd[1, :, t1]]).contiguous()
        sp = ssa().ssa_decode(qrow, kd, vd, mu, pos, wl.block, wl.top_k, ssa().SPARSE_ONLY)
        fu = ssa().ssa_decode(qrow, kd, vd, None, pos, wl.block, wl.top_k, ssa().FULL_ONLY)
        torch.cuda.synchronize()
        for b, t in ((0, t0), (1, t1)):
            ti = np.array([t])
            for h in range(wl.hq):
                c = h // wl.group
                ref_sel, _ = oracle.select_rows(qf[b, h, ti], ti, mu_ref[b, c], wl.block, wl.top_k)
                got_sel = sp["sel"][b, h].cpu().numpy()
                assert np.array_equal(got_sel, ref_sel[0]), (name, b, t, h, got_sel, ref_sel[0])
                ref = oracle.attend_rows(qf[b, h, ti], ti, kf[b, c], vf[b, c], ref_sel, wl.block, scale)
                tag = f"{name} b{b} t{t} h{h}"
                assert_close(f"{tag} h_sparse", sp["h"][b, h][None], ref["h_sparse"], wl.dtype)
                assert_close(f"{tag} lse_sparse", sp["lse"][b, h][None], ref["lse_sparse"], wl.dtype)
                assert_close(f"{tag} h_full", fu["h"][b, h][None], ref["h_full"], wl.dtype)
                assert_close(f"{tag} lse_full", fu["lse"][b, h][None], ref["lse_full"], wl.dtype)


def test_decode_equals_layer_forward_row():
    """The decode step at position t reproduces row t of the layer's
    SPARSE_ONLY and FULL_ONLY forward (same selection, outputs within the
    bf16 tolerance: different summation orders)."""
    wl = CASES["gqa_b2_n1024_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    sel = ssa().ssa_select_blocks(qd, kd, wl.block, wl.top_k)
    fs = ssa().ssa_attn_fwd(qd, kd, vd, sel, wl.block, wl.top_k, ssa().SPARSE_ONLY)
    ff = ssa().ssa_attn_fwd(qd, kd, vd, None, wl.block, wl.top_k, ssa().FULL_ONLY)
    mu = _means(kd, wl.block)
    for t in (5, 300, 1023):
        pos = torch.tensor([t, t], dtype=torch.int32, device="cuda:0")
        qrow = qd[:, :, t].contiguous()
        sp = ssa().ssa_decode(qrow, kd, vd, mu, pos, wl.block, wl.top_k, ssa().SPARSE_ONLY)
        fu = ssa().ssa_decode(qrow, kd, vd, None, pos, wl.block, wl.top_k, ssa().FULL_ONLY)
        torch.cuda.synchronize()
        assert torch.equal(sp["sel"], sel[:, :, t])
        atol, rtol = TOL[wl.dtype]
        for got, want in ((sp["h"], fs["h_sparse"][:, :, t]), (fu["h"], ff["h_full"][:, :, t]),
                          (sp["lse"], fs["lse_sparse"][:, :, t]), (fu["lse"], ff["lse_full"][:, :, t])):
            assert bool(((got.double() - want.double()).abs() <= atol + rtol * want.double().abs()).all()), t


def test_decode_top_k_one_and_all():
    """top_k 1 keeps the own block only; top_k >= blocks keeps every causal
    block, so the sparse step equals the full one."""
    wl = CASES["gqa_b2_n1024_k4"]
    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    mu = _means(kd, wl.block)
    pos = torch.tensor([700, 64], dtype=torch.int32, device="cuda:0")
    qrow = torch.stack([qd[0, :, 700], qd[1, :, 64]]).contiguous()
    one = ssa().ssa_decode(qrow, kd, vd, mu, pos, wl.block, 1, ssa().SPARSE_ONLY)
    nb = wl.seqlen // wl.block
    allk = ssa().ssa_decode(qrow, kd, vd, mu, pos, wl.block, nb, ssa().SPARSE_ONLY)
    fu = ssa().ssa_decode(qrow, kd, vd, None, pos, wl.block, nb, ssa().FULL_ONLY)
    torch.cuda.synchronize()
    assert bool((one["sel"][0, :, 0] == 700 // wl.block).all()) and bool((one["sel"][1, :, 0] == 1).all())
    own = oracle.attend_rows(qf[0, 0, [700]], np.array([700]), kf[0, 0], vf[0, 0],
                             np.array([[700 // wl.block]]), wl.block, scale_of(wl))
    assert_close("top_k 1 h", one["h"][0, 0][None], own["h_sparse"], wl.dtype)
    for b, t in ((0, 700), (1, 64)):
        want = list(range(t // wl.block + 1)) + [-1] * (nb - t // wl.block - 1)
        assert allk["sel"][b, 0].tolist() == want
    assert torch.equal(allk["lse"], fu["lse"]) or float((allk["lse"] - fu["lse"]).abs().max()) < 1e-5
    assert float((allk["h"].float() - fu["h"].float()).abs().max()) <= 2e-2


# ------------------------------------------------------------- 128K cache --

def test_decode_128k_cache_sampled_heads():
    """B=4 sequences, 16 query / 4 KV heads, a 131072-token cache with four
    planted sinks, block 64, top_k 32: decode steps at the end of the cache
    and mid-way, sampled heads against the oracle."""
    wl = W["decode_b4_n128k_sinks"]
    _say(f"decode {wl.name}: draw")
    q, k, v = si.draw_decode(wl, 0)
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    mu = _means(kd, wl.block)
    L = wl.seqlen
    pos_l = [L - 1, L // 2 + 17, 3 * wl.block + 5, L - wl.block]
    pos = torch.tensor(pos_l, dtype=torch.int32, device="cuda:0")
    sp = ssa().ssa_decode(qd, kd, vd, mu, pos, wl.block, wl.top_k, ssa().SPARSE_ONLY)
    fu = ssa().ssa_decode(qd, kd, vd, None, pos, wl.block, wl.top_k, ssa().FULL_ONLY)
    torch.cuda.synchronize()
    sel = sp["sel"].cpu().numpy()
    scale = 1.0 / math.sqrt(wl.head_dim)
    exempt = 0
    for b, h in ((0, 0), (0, 9), (1, 3), (2, 15), (3, 6)):
        c = h // wl.group
        t = pos_l[b]
        ti = np.array([t])
        kf = si.to_f64(k[b, c])
        vf = si.to_f64(v[b, c])
        qf = si.to_f64(q[b, h])[None]
        mu_c = oracle.block_means(kf[None, None], wl.block)[0, 0]
        ref_sel, margin = oracle.select_rows(qf, ti, mu_c, wl.block, wl.top_k)
        got = sel[b, h]
        if margin[0] >= 1e-3:
            assert np.array_equal(got, ref_sel[0]), (b, h, got, ref_sel[0])
        else:                                       # a valid near-optimal selection
            exempt += 1
            kept = got[got >= 0]
            i = t // wl.block
            assert kept.size == min(wl.top_k, i + 1) and kept[-1] == i and np.all(np.diff(kept) > 0)
            sigma = qf[0] @ mu_c[:i].T
            cutoff = np.sort(sigma)[::-1][min(wl.top_k - 1, i) - 1]
            assert np.all(sigma[kept[:-1]] >= cutoff - 1e-3)
        ref = oracle.attend_rows(qf, ti, kf, vf, got[None], wl.block, scale)
        tag = f"128k b{b} h{h} t{t}"
        assert_close(f"{tag} h_sparse", sp["h"][b, h][None], ref["h_sparse"], wl.dtype)
        assert_close(f"{tag} lse_sparse", sp["lse"][b, h][None], ref["lse_sparse"], wl.dtype)
        assert_close(f"{tag} h_full", fu["h"][b, h][None], ref["h_full"], wl.dtype)
        assert_close(f"{tag} lse_full", fu["lse"][b, h][None], ref["lse_full"], wl.dtype)
    _say(f"  heads exempt by margin: {exempt}")


@pytest.mark.parametrize("kind", ["zero_query", "three_levels"])
def test_decode_ties_lower_block_wins(kind):
    """Exact ties at the cutoff (scores exactly representable in fp32 and
    fp64): q = 0 ties every block; q = e_0 over block means taking three
    values ties five blocks at the top.  The lower block index must win, as
    in the oracle."""
    B, Hq, Hkv, L, d, blk, K = 2, 4, 2, 1024, 128, 64, 4
    g = torch.Generator().manual_seed(11)
    k = torch.zeros(B, Hkv, L, d)
    k[..., 0] = ((torch.arange(L) // blk) % 3).float() * 0.5      # block j: mean (j % 3) / 2 in column 0
    v = torch.randn(B, Hkv, L, d, generator=g)
    q = torch.zeros(B, Hq, d)
    if kind == "three_levels":
        q[..., 0] = 1.0
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    mu = _means(kd, blk)
    pos_l = [L - 1, 9 * blk + 3]
    pos = torch.tensor(pos_l, dtype=torch.int32, device="cuda:0")
    sp = ssa().ssa_decode(qd, kd, vd, mu, pos, blk, K, ssa().SPARSE_ONLY)
    torch.cuda.synchronize()
    kf, vf, qf = si.to_f64(k), si.to_f64(v), si.to_f64(q)
    for b in range(B):
        t = pos_l[b]
        ti = np.array([t])
        for h in range(Hq):
            c = h // (Hq // Hkv)
            mu_c = oracle.block_means(kf[b:b + 1, c:c + 1], blk)[0, 0]
            ref_sel, _ = oracle.select_rows(qf[b, h][None], ti, mu_c, blk, K)
            assert sp["sel"][b, h].tolist() == ref_sel[0].tolist(), (kind, b, h)
            ref = oracle.attend_rows(qf[b, h][None], ti, kf[b, c], vf[b, c], ref_sel, blk, 1.0 / math.sqrt(d))
            assert_close(f"ties {kind} b{b} h{h}", sp["h"][b, h][None], ref["h_sparse"], torch.bfloat16)


# --------------------------------------------------------- chunked prefill --

@pytest.mark.parametrize("name", ["gqa_b2_n1024_k4", "mha_b2_n512_b32_k6", "gqa_b2_n768_b128_k3"])
def test_prefill_chunks_equal_layer_rows(name):
    """Chunks of a prompt processed against the cache reproduce the layer's
    rows: the same selection (bit for bit) and both streams, and the oracle's
    rows on a sample."""
    wl = CASES[name]
    _say(f"prefill {name}")
    (q, k, v), (qf, kf, vf) = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    N, blk, K = wl.seqlen, wl.block, wl.top_k
    sel = ssa().ssa_select_blocks(qd, kd, blk, K)
    fs = ssa().ssa_attn_fwd(qd, kd, vd, sel, blk, K, ssa().SPARSE_ONLY)
    ff = ssa().ssa_attn_fwd(qd, kd, vd, None, blk, K, ssa().FULL_ONLY)
    mu = _means(kd, blk)
    mu_ref = oracle.block_means(kf, blk)
    scale = scale_of(wl)
    chunks = [(0, 2 * blk), (2 * blk, N // 2 - 2 * blk), (N // 2, blk), (N // 2 + blk, N // 2 - blk)]
    rng = np.random.default_rng(8)
    for p0, C in chunks:
        qc = qd[:, :, p0:p0 + C].contiguous()
        sp = ssa().ssa_prefill(qc, kd, vd, mu, p0, blk, K, ssa().SPARSE_ONLY)
        fu = ssa().ssa_prefill(qc, kd, vd, None, p0, blk, K, ssa().FULL_ONLY)
        torch.cuda.synchronize()
        tag = f"{name} chunk {p0}+{C}"
        assert torch.equal(sp["sel"], sel[:, :, p0:p0 + C]), tag
        atol, rtol = TOL[wl.dtype]
        for got, want in ((sp["h"], fs["h_sparse"][:, :, p0:p0 + C]), (sp["lse"], fs["lse_sparse"][:, :, p0:p0 + C]),
                          (fu["h"], ff["h_full"][:, :, p0:p0 + C]), (fu["lse"], ff["lse_full"][:, :, p0:p0 + C])):
            diff = (got.double() - want.double()).abs() - (atol + rtol * want.double().abs())
            assert float(diff.max()) <= 0, tag
        # a sample of the chunk's rows against the oracle
        for b in range(wl.batch):
            h = int(rng.integers(0, wl.hq))
            c = h // wl.group
            rows = np.unique(np.concatenate([[0, C - 1], rng.integers(0, C, size=4)]))
            ti = p0 + rows
            ref_sel, _ = oracle.select_rows(qf[b, h, ti], ti, mu_ref[b, c], blk, K)
            assert np.array_equal(sp["sel"][b, h, torch.from_numpy(rows)].cpu().numpy(), ref_sel), tag
            ref = oracle.attend_rows(qf[b, h, ti], ti, kf[b, c], vf[b, c], ref_sel, blk, scale)
            idx = torch.from_numpy(rows)
            assert_close(f"{tag} b{b} h{h} h_sparse", sp["h"][b, h, idx], ref["h_sparse"], wl.dtype)
            assert_close(f"{tag} b{b} h{h} lse_sparse", sp["lse"][b, h, idx], ref["lse_sparse"], wl.dtype)
            assert_close(f"{tag} b{b} h{h} h_full", fu["h"][b, h, idx], ref["h_full"], wl.dtype)
            assert_close(f"{tag} b{b} h{h} lse_full", fu["lse"][b, h, idx], ref["lse_full"], wl.dtype)


def test_prefill_argument_errors():
    wl = CASES["gqa_b2_n1024_k4"]
    (q, k, v), _ = inputs(wl, 0, (wl.top_k,))
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    mu = _means(kd, wl.block)
    with pytest.raises(ssa().SSAError):          # chunk past the cache
        ssa().ssa_prefill(qd[:, :, :128].contiguous(), kd, vd, mu, 1024 - 64, wl.block, wl.top_k)
    with pytest.raises(ssa().SSAError):          # position not on a block boundary
        ssa().ssa_prefill(qd[:, :, :128].contiguous(), kd, vd, mu, 32, wl.block, wl.top_k)
    with pytest.raises(ssa().SSAError):          # dual modes are training modes
        ssa().ssa_prefill(qd[:, :, :128].contiguous(), kd, vd, mu, 0, wl.block, wl.top_k, ssa().DUAL_ACTIVE_FULL)


def test_prefill_then_decode_128k_sampled():
    """A 4096-token chunk near the end of a 131072-token prompt (B=4, 16/4
    heads, top_k 32, sinks), sparse and full, on sampled rows against the
    oracle; then one decode step per sequence at the positions right after
    the chunk, against the oracle's rows.  Near-ties (fp64 cutoff margin below
    1e-3) are exempt from equality, and their selection must be a valid
    near-optimal one."""
    wl = W["decode_b4_n128k_sinks"]
    _say(f"prefill {wl.name}: draw")
    q_dec, k, v = si.draw_decode(wl, 0)
    g = torch.Generator().manual_seed(21)
    C, L, blk, K = 4096, wl.seqlen, wl.block, wl.top_k
    p0 = L - C - 2 * blk            # positions p0 .. p0 + C - 1; decode right after
    qc = torch.randn(wl.batch, wl.hq, C, wl.head_dim, generator=g).to(torch.bfloat16)
    qd, kd, vd = (x.to("cuda:0") for x in (qc, k, v))
    mu = _means(kd, blk)
    sp = ssa().ssa_prefill(qd, kd, vd, mu, p0, blk, K, ssa().SPARSE_ONLY)
    fu = ssa().ssa_prefill(qd, kd, vd, None, p0, blk, K, ssa().FULL_ONLY)
    # decode: sequence b at position p0 + C + 37 b (the last inside the next block
    # for b = 3, 3 * 37 = 111 < 2 * 64): keys up to it are in the cache
    pos_np = np.array([p0 + C + 37 * b for b in range(wl.batch)], dtype=np.int32)
    pos = torch.from_numpy(pos_np).to("cuda:0")
    qdd = q_dec.to("cuda:0")
    dsp = ssa().ssa_decode(qdd, kd, vd, mu, pos, blk, K, ssa().SPARSE_ONLY)
    dfu = ssa().ssa_decode(qdd, kd, vd, None, pos, blk, K, ssa().FULL_ONLY)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(wl.head_dim)
    rng = np.random.default_rng(5)
    exempt = 0
    for b, h in ((0, 2), (3, 13), (1, 7)):
        c = h // wl.group
        kf, vf = si.to_f64(k[b, c]), si.to_f64(v[b, c])
        mu_c = oracle.block_means(kf[None, None], blk)[0, 0]
        rows = np.unique(np.concatenate([[0, blk - 1, C - 1], rng.integers(0, C, size=5)]))
        ti = p0 + rows
        qf = si.to_f64(qc[b, h])[rows]
        got = sp["sel"][b, h, torch.from_numpy(rows)].cpu().numpy()
        exempt += check_selection(f"128k prefill b{b} h{h}", qf, ti, mu_c, blk, K, got)
        ref = oracle.attend_rows(qf, ti, kf, vf, got, blk, scale)
        idx = torch.from_numpy(rows)
        tag = f"128k prefill b{b} h{h}"
        assert_close(f"{tag} h_sparse", sp["h"][b, h, idx], ref["h_sparse"], wl.dtype)
        assert_close(f"{tag} lse_sparse", sp["lse"][b, h, idx], ref["lse_sparse"], wl.dtype)
        assert_close(f"{tag} h_full", fu["h"][b, h, idx], ref["h_full"], wl.dtype)
        assert_close(f"{tag} lse_full", fu["lse"][b, h, idx], ref["lse_full"], wl.dtype)
        # the decode step of this sequence and head
        t = np.array([pos_np[b]])
        qrow = si.to_f64(q_dec[b, h])[None]
        dsel = dsp["sel"][b, h].cpu().numpy()[None]
        exempt += check_selection(f"128k decode b{b} h{h}", qrow, t, mu_c, blk, K, dsel)
        dref = oracle.attend_rows(qrow, t, kf, vf, dsel, blk, scale)
        tag = f"128k decode b{b} h{h} t{int(t[0])}"
        assert_close(f"{tag} h_sparse", dsp["h"][b, h][None], dref["h_sparse"], wl.dtype)
        assert_close(f"{tag} lse_sparse", dsp["lse"][b, h][None], dref["lse_sparse"], wl.dtype)
        assert_close(f"{tag} h_full", dfu["h"][b, h][None], dref["h_full"], wl.dtype)
        assert_close(f"{tag} lse_full", dfu["lse"][b, h][None], dref["lse_full"], wl.dtype)
    _say(f"  rows exempt by margin: {exempt}")
