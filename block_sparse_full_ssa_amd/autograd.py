"""torch.autograd binding of one SSA attention layer.

SSA trains each layer in two streams over the same q, k, v (Sintesi Tecnica,
section 2): the active stream's output goes on to the rest of the network,
the counterpart output exists only for the alignment losses.  L_sparsity
pulls h_full toward a fixed h_sparse and L_commit pulls h_sparse toward a
fixed h_full, so in the backward the upstream gradient reaches the active
output only, and each loss reaches only the output it moves.

``SSAFunction`` wraps ssa_attn_fwd / ssa_attn_bwd (argument marshalling only;
the library does every step).  Its outputs are

  h       the active output [B, Hq, N, d] (h_full for DUAL_ACTIVE_FULL and
          FULL_ONLY, h_sparse for DUAL_ACTIVE_SPARSE and SPARSE_ONLY);
  losses  float32 [2] = (L_sparsity, L_commit) in the dual modes (equal values),
          zeros in the single-stream modes (no gradient flows from them there);
  delta   float32 [B, Hq, N], the discarded mass (dual modes; empty otherwise).

The counterpart output is kept for the backward only.  The gradient of
``losses`` gives the weights w_sparsity and w_commit of the library's
backward; reading them is one small device-to-host copy, taken only when some
loss is part of the differentiated objective.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

import torch

from ._lib import DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY
from . import ops

_FULL_ACTIVE = (DUAL_ACTIVE_FULL, FULL_ONLY)
_DUAL = (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE)


class SSAFunction(torch.autograd.Function):
    """(h_active, losses, delta) = SSAFunction.apply(q, k, v, sel, block, top_k, mode, scale)."""

    @staticmethod
    def forward(ctx, q, k, v, sel, block: int, top_k: int, mode: int, scale: Optional[float]):
        if mode not in (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY):
            raise ValueError(f"unknown mode {mode}")
        fwd = ops.ssa_attn_fwd(q, k, v, sel, block, top_k, mode, scale)
        dual = mode in _DUAL
        h = fwd["h_full"] if mode in _FULL_ACTIVE else fwd["h_sparse"]
        if dual:
            losses, delta = fwd["losses"], fwd["delta"]
        else:
            losses = torch.zeros(2, dtype=torch.float32, device=q.device)
            delta = torch.empty(0, dtype=torch.float32, device=q.device)
        names = [n for n in ("h_full", "h_sparse", "lse_full", "lse_sparse") if n in fwd]
        ctx.names = names
        ctx.cfg = (block, top_k, mode, scale)
        ctx.has_sel = sel is not None
        ctx.save_for_backward(q, k, v, sel if sel is not None else q.new_empty(0), *(fwd[n] for n in names))
        ctx.mark_non_differentiable(delta)
        if not dual:
            ctx.mark_non_differentiable(losses)
        return h, losses, delta

    @staticmethod
    def backward(ctx, g_h, g_losses, g_delta):
        q, k, v, sel, *saved = ctx.saved_tensors
        block, top_k, mode, scale = ctx.cfg
        fwd = dict(zip(ctx.names, saved))
        w_s = w_c = 0.0
        if mode in _DUAL and g_losses is not None:
            w_s, w_c = (float(x) for x in g_losses.detach().float().cpu())
        d_out = g_h.contiguous() if g_h is not None else None
        dq, dk, dv = ops.ssa_attn_bwd(q, k, v, sel if ctx.has_sel else None, fwd, d_out, block, top_k, mode,
                                      w_s, w_c, scale)
        return dq, dk, dv, None, None, None, None, None


class SSAOutput(NamedTuple):
    h: torch.Tensor          # the active output
    losses: torch.Tensor     # (L_sparsity, L_commit)
    delta: torch.Tensor      # discarded mass per query (dual modes)
    sel: Optional[torch.Tensor]


def ssa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int, top_k: int,
                  mode: int = DUAL_ACTIVE_FULL, sel: Optional[torch.Tensor] = None,
                  scale: Optional[float] = None) -> SSAOutput:
    """One SSA layer with autograd: selects the blocks (unless ``sel`` is given;
    FULL_ONLY needs none), runs the forward, and returns the active output,
    the alignment losses, delta and the selection.  Backpropagating
    ``<dO, h> + a L_sparsity + c L_commit`` gives the library's backward with
    d_out = dO, w_sparsity = a and w_commit = c."""
    if sel is None and mode != FULL_ONLY:
        sel = ops.ssa_select_blocks(q.detach(), k.detach(), block, top_k)
    h, losses, delta = SSAFunction.apply(q, k, v, sel, int(block), int(top_k), int(mode), scale)
    return SSAOutput(h, losses, delta, sel)
