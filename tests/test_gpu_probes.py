"""The machine probes behind the measured ceilings: the copy probe moves bytes
exactly (including a ragged tail), and the matrix-core probe runs at a rate
between a tenth of the datasheet bf16 peak and that peak."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_copy_exact_with_ragged_tail():
    import block_sparse_full_ssa_amd as ssa
    g = torch.Generator(device="cpu").manual_seed(7)
    n = (64 << 20) // 4 + 12            # 64 MiB + 48 bytes: not a whole number of 16 KiB blocks
    src = torch.randint(-2**31, 2**31 - 1, (n,), generator=g, dtype=torch.int32).cuda()
    dst = torch.zeros_like(src)
    ssa.ssa_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # a copy shorter than one lane's vector set leaves the rest untouched
    dst2 = torch.zeros(64, dtype=torch.int32, device="cuda")
    ssa.ssa_probe_copy(src[:4], dst2)
    torch.cuda.synchronize()
    assert torch.equal(dst2[:4], src[:4]) and int(dst2[4:].abs().sum()) == 0


def test_probe_mfma_rate_plausible():
    import block_sparse_full_ssa_amd as ssa
    blocks, iters = 512, 2000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ssa.ssa_probe_mfma(sink, blocks, 50)          # warm-up
    torch.cuda.synchronize()
    ssa.timing_enable(True)
    ssa.ssa_probe_mfma(sink, blocks, iters)
    ms, n = ssa.timing_query("probe_mfma")
    ssa.timing_enable(False)
    assert n == 1 and ms > 0
    tflops = blocks * 16 * iters * 32768 / (ms / 1e3) / 1e12
    assert 250.0 < tflops < 2600.0, tflops
    assert torch.isfinite(sink).all()


def test_probe_atomic_counts_exact():
    """Every float of every tile is incremented exactly (workgroups per tile) x iters times."""
    import block_sparse_full_ssa_amd as ssa
    ntiles, blocks, iters = 64, 512, 16
    buf = torch.zeros(ntiles * 4096, dtype=torch.float32, device="cuda")
    ssa.timing_enable(True)
    ssa.ssa_probe_atomic(buf, blocks, iters)
    ms, n = ssa.timing_query("probe_atomic")
    ssa.timing_enable(False)
    assert n == 1 and ms > 0
    assert bool((buf == float(blocks // ntiles * iters)).all())


@pytest.mark.parametrize("mode", list(range(10)))
def test_probe_lds_runs(mode):
    import block_sparse_full_ssa_amd as ssa
    blocks = 512
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ssa.timing_enable(True)
    ssa.ssa_probe_lds(sink, blocks, 200, mode)
    ms, n = ssa.timing_query("probe_lds")
    ssa.timing_enable(False)
    assert n == 1 and ms > 0 and torch.isfinite(sink).all()
