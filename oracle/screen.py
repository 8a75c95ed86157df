"""Near-tie screening of query rows for exact selection parity.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

A GPU computes block scores with fp32 sums (and bf16 layers with the means
split into two bf16 terms) and the oracle in fp64, so a row whose top-k
cutoff separates two scores closer than that rounding could be ranked
differently.  Rows whose cutoff margin (the oracle's fp64 score of
the last kept block minus that of the first dropped block) is below the
threshold are redrawn from the same seeded stream, in (batch, head, token)
order, until no row fails at any of the given top-k values.  k and v are
never redrawn.  Returns the screened q and the number of redrawn rows.
"""
from __future__ import annotations

import numpy as np
import torch

import ssa_inputs
from .ssa_oracle import block_means, select_rows


def screen_q(q: torch.Tensor, k: torch.Tensor, block: int, top_ks, group: int,
             gen: torch.Generator, prescale: float = 1.0, threshold: float = 1e-3,
             max_rounds: int = 200):
    top_ks = [top_ks] if isinstance(top_ks, int) else list(top_ks)
    B, Hq, N, d = q.shape
    q = q.clone()
    mu = block_means(ssa_inputs.to_f64(k), block)
    redrawn = 0
    for b in range(B):
        for h in range(Hq):
            rows = np.arange(N)
            for _ in range(max_rounds):
                qf = ssa_inputs.to_f64(q[b, h, rows])
                bad = np.zeros(rows.size, dtype=bool)
                for kk in top_ks:
                    _, margin = select_rows(qf, rows, mu[b, h // group], block, kk)
                    bad |= margin < threshold
                rows = rows[bad]
                if rows.size == 0:
                    break
                q[b, h, torch.from_numpy(rows)] = ssa_inputs.redraw_rows(
                    gen, rows.size, d, q.dtype, prescale)
                redrawn += rows.size
            else:
                raise RuntimeError("screening did not converge")
    return q, redrawn
