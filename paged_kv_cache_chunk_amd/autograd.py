"""PyTorch autograd view of one chunk's paged attention.

The paged KV cache is not an autograd input: the forward reads K/V from the
pool, and the backward adds dK/dV straight into the pool's gradient pages
("Out of the Memory Barrier", gist.science de, sections 2.A and 2.B;
sciencestack.ai, Figure 3), so only q receives a gradient through autograd.
Both directions are libpkv calls on the current stream; this module only
allocates the outputs and marshals arguments.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import Pool, pkv_attn_bwd, pkv_attn_fwd


class PagedAttention(torch.autograd.Function):
    """o = PagedAttention.apply(q, pool, layer, q_pos0, scale, sel)

    q: [n_q][Hq][d] device tensor in the pool's K/V dtype; sel: None (dense
    causal) or the (pages, count) selection of the chunk, held constant.
    Returns o (q's dtype).  Backward: q.grad (q's dtype; libpkv computes it in
    fp32) and dK, dV added into the pool for `layer`.  The log-sum-exp of the
    forward is kept for the backward, which recomputes the probabilities.
    """

    @staticmethod
    def forward(ctx, q: torch.Tensor, pool: Pool, layer: int, q_pos0: int, scale: float,
                sel: Optional[tuple] = None) -> torch.Tensor:
        q = q.contiguous()
        n_q, hq, _ = q.shape
        o = torch.empty_like(q)
        lse = torch.empty(hq, n_q, dtype=torch.float32, device=q.device)
        pkv_attn_fwd(pool, layer, q_pos0, q, o, lse, scale, sel=sel)
        ctx.save_for_backward(q, o, lse)
        ctx.pool, ctx.layer, ctx.q_pos0, ctx.scale, ctx.sel = pool, layer, q_pos0, scale, sel
        return o

    @staticmethod
    def backward(ctx, do: torch.Tensor):
        q, o, lse = ctx.saved_tensors
        do = do.to(q.dtype).contiguous()
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        pkv_attn_bwd(ctx.pool, ctx.layer, ctx.q_pos0, q, o, do, lse, dq, ctx.scale, sel=ctx.sel)
        return dq.to(q.dtype), None, None, None, None, None


def paged_attention(q: torch.Tensor, pool: Pool, layer: int, q_pos0: int, scale: float,
                    sel: Optional[tuple] = None) -> torch.Tensor:
    """Functional form of PagedAttention.apply."""
    return PagedAttention.apply(q, pool, layer, q_pos0, scale, sel)
