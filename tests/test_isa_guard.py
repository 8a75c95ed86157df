"""Compiled-code guard (CPU, needs hipcc): no MFMA and no transposing LDS read
issued under a narrowed EXEC."""
import pytest

from block_sparse_full_ssa_amd import isa_check


def test_scanner_flags_masked_mfma():
    asm = "\n".join([
        "s_and_saveexec_b64 s[4:5], s[34:35]",
        "v_mfma_f32_32x32x16_bf16 a[48:63], v[20:23], v[128:131], a[48:63]",
        "s_or_b64 exec, exec, s[4:5]",
        "s_and_saveexec_b64 s[4:5], s[34:35]",
        "s_cbranch_execz .LBB2_77",
        "v_mfma_f32_32x32x16_bf16 a[112:127], v[20:23], v[128:131], a[112:127]",
    ])
    hits = isa_check.masked_mfmas(asm)
    assert [ln for ln, _ in hits] == [1]
    # a block label (even with a trailing comment) ends the backward scan
    asm2 = "\n".join([
        "s_and_saveexec_b64 s[4:5], s[34:35]",
        ".LBB2_60:                               ;   in Loop: Header=BB2_39 Depth=1",
        "v_mfma_f32_32x32x16_bf16 v[144:159], v[198:201], a[44:47], v[144:159]",
    ])
    assert isa_check.masked_mfmas(asm2) == []


def test_scanner_flags_masked_transpose():
    asm = "\n".join([
        "ds_read_b64_tr_b16 v[66:67], v72",
        "s_and_saveexec_b64 s[4:5], vcc",
        "s_cbranch_execz .LBB10_31",
        "ds_read_b64_tr_b16 v[68:69], v72 offset:512",
        "s_or_b64 exec, exec, s[4:5]",
        "ds_read_b64_tr_b16 v[70:71], v72 offset:1024",
    ])
    # a partial EXEC is wrong even behind an execz branch
    assert [ln for ln, _ in isa_check.masked_transposes(asm)] == [3]


@pytest.mark.parametrize("src", isa_check.MFMA_SOURCES)
def test_no_masked_transpose_in_kernels(src):
    import os
    from block_sparse_full_ssa_amd import build
    if not os.path.exists(os.path.join(build.CSRC, src)):
        pytest.skip(f"{src} not present")
    assert isa_check.masked_transposes(isa_check.device_asm(src)) == []


@pytest.mark.parametrize("src", isa_check.MFMA_SOURCES)
def test_no_masked_mfma_in_kernels(src):
    import os
    from block_sparse_full_ssa_amd import build
    if not os.path.exists(os.path.join(build.CSRC, src)):
        pytest.skip(f"{src} not present")
    asm = isa_check.device_asm(src)
    if "v_mfma" not in asm:
        pytest.skip(f"{src} has no MFMA")
    assert isa_check.masked_mfmas(asm) == []
