"""Builds libssa.so (the HIP kernels and the C entry points) for gfx950.

Each .hip source is compiled to an object in parallel with hipcc, then the
objects are linked into a shared library next to this file.  Every call
compiles from scratch.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libssa.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.hip", "select.hip", "simt.hip", "misc.hip", "fwd_mfma.hip", "bwd_mfma.hip", "bucket.hip",
           "sparse_fwd.hip", "sparse_bwd.hip", "bwd_dq.hip", "probe.hip", "decode.hip", "static_ws.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-munsafe-fp-atomics",
    # keep MFMA accumulators in VGPRs where they fit (no AGPR round trips)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source flags.  The forward kernel takes running maxima of matrix
# products: without NaN semantics (no NaN arises from finite inputs there:
# masked logits are -inf and every row's running maximum is finite from its
# first key tile on) the compiler emits max instructions without quieting
# each operand first, and the IEEE mode bit is off for its kernels.
FILE_FLAGS = {
    "fwd_mfma.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def flags_for(src: str) -> list:
    return [*HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libssa")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
