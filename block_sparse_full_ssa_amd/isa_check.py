"""Static checks of the compiled gfx950 code for two instruction classes that
combine the data of all 64 lanes and so must not run under a narrowed EXEC.

The compiler implements an `if` whose condition it believes to be per-lane by
masking EXEC.  Matrix (MFMA) instructions were observed to run even under
EXEC = 0 in that form, adding stale operands to accumulators: kernels make
every MFMA guard wave-uniform (readfirstlane), and the check fails if an MFMA
follows an EXEC-narrowing instruction without an execz branch between.
Transposing LDS reads (ds_read_b64_tr_b16) hand each lane data that other
lanes read, so under a partial EXEC they return unread data: the check fails
on any such read after an EXEC-narrowing instruction.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build as _build

_NARROW = re.compile(r"^(s_and_saveexec|s_andn2_saveexec|s_and_b64 exec|s_andn2_b64 exec|s_xor_b64 exec)")
_EXEC_WRITE = re.compile(r"^(s_and_saveexec|s_andn2_saveexec|s_or_saveexec|s_and_b64 exec|s_andn2_b64 exec|"
                         r"s_mov_b64 exec|s_or_b64 exec|s_xor_b64 exec)")


def masked_mfmas(asm: str):
    """(line number, instruction) of every MFMA issued under a narrowed EXEC."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    found = []
    for i, t in enumerate(lines):
        if not t.startswith("v_mfma"):
            continue
        j, guarded = i - 1, False
        while j >= 0:
            u = lines[j]
            if u.startswith("s_cbranch_execz"):
                guarded = True
            if _EXEC_WRITE.match(u) or (u.startswith(".LBB") and u.endswith(":")):
                break
            j -= 1
        if j >= 0 and _NARROW.match(lines[j]) and not guarded:
            found.append((i, t))
    return found


def masked_transposes(asm: str):
    """(line number, instruction) of every transposing LDS read issued under a
    narrowed EXEC (guarded by an execz branch or not)."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    found = []
    for i, t in enumerate(lines):
        if not re.match(r"ds_read_b\d+_tr", t):
            continue
        j = i - 1
        while j >= 0:
            u = lines[j]
            if _EXEC_WRITE.match(u) or (u.startswith(".LBB") and u.endswith(":")):
                break
            j -= 1
        if j >= 0 and _NARROW.match(lines[j]):
            found.append((i, t))
    return found


def device_asm(source: str) -> str:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [_build.hipcc(), *_build.flags_for(source), "-S", "--cuda-device-only",
               os.path.join(_build.CSRC, source), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed on {source}:\n{r.stderr}")
        return open(out).read()


MFMA_SOURCES = ("select.hip", "fwd_mfma.hip", "bwd_mfma.hip", "sparse_fwd.hip", "sparse_bwd.hip", "bwd_dq.hip")


def main() -> int:
    bad = 0
    for src in MFMA_SOURCES:
        if not os.path.exists(os.path.join(_build.CSRC, src)):
            continue
        asm = device_asm(src)
        hits = masked_mfmas(asm) + masked_transposes(asm)
        for ln, ins in hits[:5]:
            print(f"{src}: asm line {ln}: {ins}", file=sys.stderr)
        bad += len(hits)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
