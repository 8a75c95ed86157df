"""Seeded synthetic inputs for SSA dual-stream attention.

This module only draws random numbers and shapes them; it contains none of
the attention arithmetic.  Both the CPU oracle (through its tests and the
screening helper) and the GPU path (through the tests and the benchmark) take
their inputs from here, so the two sides always see the same tensors.

The workloads stand in for a trained model's per-layer q/k/v activations; the
pages measure on language-model suites (commonsense, needle retrieval,
LongBench) that carry no attention tensors, so i.i.d. Gaussian activations of
the stated shapes are used instead.  Every draw is from a CPU
``torch.Generator`` so that the same seed gives the same bits on any machine.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer shape.  ``hq`` query heads share ``hkv`` KV heads."""

    name: str
    batch: int
    hq: int
    hkv: int
    seqlen: int
    head_dim: int
    block: int
    top_k: int
    dtype: torch.dtype
    # q/k/v are N(0, 1) draws multiplied by this factor before rounding to
    # ``dtype`` (the tiny fp32 layer draws N(0,1)/sqrt(d)).
    prescale: float = 1.0
    # high-norm keys planted at positions 0..n_sinks-1 of every KV head
    n_sinks: int = 0
    layers: int = 1
    top_k_sweep: tuple = ()

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def nblocks(self) -> int:
        return self.seqlen // self.block


def _wl(**kw) -> Workload:
    return Workload(**kw)


# The layer shapes the measurements are quoted on, and the decode cache (128K).
WORKLOADS: Dict[str, Workload] = {
    "tiny_mha_n256_fp32": _wl(
        name="tiny_mha_n256_fp32", batch=1, hq=2, hkv=2, seqlen=256, head_dim=64,
        block=32, top_k=4, dtype=torch.float32, prescale=1.0 / math.sqrt(64)),
    "gqa_n4k_fwd": _wl(
        name="gqa_n4k_fwd", batch=1, hq=16, hkv=4, seqlen=4096, head_dim=128,
        block=64, top_k=16, dtype=torch.bfloat16),
    "train_b2_h32_n16k": _wl(
        name="train_b2_h32_n16k", batch=2, hq=32, hkv=8, seqlen=16384, head_dim=128,
        block=64, top_k=16, dtype=torch.bfloat16, top_k_sweep=(4, 8, 16, 32)),
    "long_n64k_sinks": _wl(
        name="long_n64k_sinks", batch=1, hq=16, hkv=4, seqlen=65536, head_dim=128,
        block=64, top_k=32, dtype=torch.bfloat16, n_sinks=4),
    "decode_b4_n128k_sinks": _wl(
        name="decode_b4_n128k_sinks", batch=4, hq=16, hkv=4, seqlen=131072, head_dim=128,
        block=64, top_k=32, dtype=torch.bfloat16, n_sinks=4),
    "multilayer_b4_n8k_l4": _wl(
        name="multilayer_b4_n8k_l4", batch=4, hq=32, hkv=8, seqlen=8192, head_dim=128,
        block=64, top_k=16, dtype=torch.bfloat16, layers=4),
}


def generator(seed: int, device: str = "cpu") -> torch.Generator:
    """A seeded torch generator.  The tests draw on the CPU (the same bits on
    any machine); the benchmark may draw its largest layers on the GPU
    (seeded too, but another stream of numbers than the CPU's)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw(gen: torch.Generator, shape, dtype: torch.dtype, prescale: float = 1.0) -> torch.Tensor:
    """N(0, 1) * prescale, rounded (round-to-nearest-even) to ``dtype``, on the
    generator's device."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)
    if prescale != 1.0:
        x = x * prescale
    return x.to(dtype)


def draw_qkv(wl: Workload, seed: int, layer: int = 0, device: str = "cpu"):
    """q [B,Hq,N,d], k and v [B,Hkv,N,d], drawn in that order from one stream.

    Also returns the generator, positioned after the last draw, so that a
    screening pass can keep redrawing query rows from the same stream.
    """
    gen = generator(seed + 1000 * layer, device)
    B, N, d = wl.batch, wl.seqlen, wl.head_dim
    q = draw(gen, (B, wl.hq, N, d), wl.dtype, wl.prescale)
    k = draw(gen, (B, wl.hkv, N, d), wl.dtype, wl.prescale)
    v = draw(gen, (B, wl.hkv, N, d), wl.dtype, wl.prescale)
    if wl.n_sinks:
        k = plant_sinks(k, gen, wl.n_sinks)
    return q, k, v, gen


def draw_decode(wl: Workload, seed: int, device: str = "cpu"):
    """A decode step's inputs: caches k, v [B,Hkv,N,d] (N = the cache's
    capacity) and one query row per sequence and head, q [B,Hq,d], drawn in
    the order k, v, q from stream seed + 3 (sinks planted as for a layer)."""
    gen = generator(seed + 3, device)
    B, N, d = wl.batch, wl.seqlen, wl.head_dim
    k = draw(gen, (B, wl.hkv, N, d), wl.dtype, wl.prescale)
    v = draw(gen, (B, wl.hkv, N, d), wl.dtype, wl.prescale)
    q = draw(gen, (B, wl.hq, d), wl.dtype, wl.prescale)
    if wl.n_sinks:
        k = plant_sinks(k, gen, wl.n_sinks)
    return q, k, v


def plant_sinks(k: torch.Tensor, gen: torch.Generator, n_sinks: int) -> torch.Tensor:
    """Add 8*sqrt(d)*u_c to keys 0..n_sinks-1 of KV head c (u_c: seeded unit vector).

    The pages report that attention over-allocates mass to sink positions
    (abstract); these planted high-norm keys give logits far above the rest.
    """
    B, H, N, d = k.shape
    u = torch.randn(B, H, d, generator=gen, dtype=torch.float32, device=gen.device)
    u = u / u.norm(dim=-1, keepdim=True)
    kf = k.float()
    kf[:, :, :n_sinks, :] += (8.0 * math.sqrt(d)) * u[:, :, None, :]
    return kf.to(k.dtype)


def redraw_rows(gen: torch.Generator, count: int, d: int, dtype: torch.dtype,
                prescale: float = 1.0) -> torch.Tensor:
    """``count`` fresh query rows of width ``d`` from the same stream."""
    return draw(gen, (count, d), dtype, prescale)


def draw_dout(wl: Workload, seed: int, layer: int = 0, device: str = "cpu") -> torch.Tensor:
    """Upstream gradient of the active output, N(0,1), [B,Hq,N,d], stream seed+1."""
    gen = generator(seed + 1 + 1000 * layer, device)
    return draw(gen, (wl.batch, wl.hq, wl.seqlen, wl.head_dim), wl.dtype)


def draw_modes(seed: int, steps: int) -> List[int]:
    """Active stream per training step, 0 = full, 1 = sparse, each with p = 1/2.

    Drawn once per step from stream seed+2 and shared by every layer of that
    step (Sintesi Tecnica, section 2 'Meccanismo Core': one of the two modes is
    picked uniformly at random at each training step).
    """
    gen = generator(seed + 2)
    return [int(x) for x in torch.randint(0, 2, (steps,), generator=gen)]


def scaled_down(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with some fields changed (smaller parity cases)."""
    d = dataclasses.asdict(wl)
    d.update(changes)
    return Workload(**d)


def to_f64(x: torch.Tensor):
    """Exact conversion of a CPU tensor (fp32 or bf16) to a float64 numpy array."""
    return x.detach().to("cpu").to(torch.float64).numpy()
