"""Chunk-recurrent training of one attention block over the paged KV cache.

The setting the library is built for ("Out of the Memory Barrier",
gist.science de, sections 2.A and 2.B; sciencestack.ai, Figure 3): a long
sequence is processed in query chunks.  The forward sweep runs chunk by chunk
without autograd and only appends each chunk's K/V to the paged cache.  The
backward sweep runs the chunks last to first; for each chunk it recomputes
the chunk's block with autograd, with attention over the paged cache as an
opaque op whose backward adds the chunk's dK/dV into the pool's gradient
pages.  By the time the sweep reaches a chunk, every later chunk has added
its contribution, so the chunk's own K/V gradients are complete: they are
read from the pool and carried back through the chunk's K/V projections.
Activation memory is that of one chunk whatever the context length; the
context costs only the pool's pages.

The block is y = x + W_o attn(RoPE(W_q x), RoPE(W_k x), W_v x) with grouped
query heads, random-initialised (no trained weights are involved).  Matrix
products are torch's (BLAS); attention, selection and the KV-gradient
accumulation are libpkv calls.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import (PKV_BF16, PKV_DK, PKV_DV, PKV_F32, pkv_append_kv, pkv_grad_zero, pkv_pool_create,
               pkv_pool_reset, pkv_read_rows, pkv_select_topk_pages)
from .autograd import paged_attention
from .chunks import Sparse


class AttentionBlock:
    """One attention block trained chunk-recurrently.

    hidden, hq, hkv, d: the block's shape (Qwen2.5-7B: 3584, 28, 4, 128).
    max_tokens: context capacity of the pool (pages of `page` tokens).
    sparse: None (dense causal) or a Sparse top-K budget.
    Weights are fp32 master copies (requires_grad) used in `dtype` (bf16)
    products; the pool holds K/V in `dtype` and gradients in fp32.
    """

    def __init__(self, hidden: int = 3584, hq: int = 28, hkv: int = 4, d: int = 128,
                 rope_base: float = 1e6, page: int = 128, max_tokens: int = 131072,
                 sparse: Optional[Sparse] = None, dtype: torch.dtype = torch.bfloat16,
                 seed: int = 0, device: str = "cuda"):
        self.hidden, self.hq, self.hkv, self.d = hidden, hq, hkv, d
        self.page, self.sparse, self.dtype, self.device = page, sparse, dtype, device
        self.rope_base = rope_base
        self.scale = d ** -0.5
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def w(rows, cols):
            return (torch.randn(rows, cols, generator=g, device=device) * 0.02).requires_grad_()
        self.wq, self.wk = w(hq * d, hidden), w(hkv * d, hidden)
        self.wv, self.wo = w(hkv * d, hidden), w(hidden, hq * d)
        pages = -(-max_tokens // page)
        kvd = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
        self.pool = pkv_pool_create(1, hkv, d, page, pages, pages, kvd)
        half = d // 2
        self._inv = rope_base ** (-torch.arange(half, dtype=torch.float64, device=device) * 2.0 / d)

    def parameters(self) -> List[torch.Tensor]:
        return [self.wq, self.wk, self.wv, self.wo]

    # ---- pieces of the block
    def _rope(self, x: torch.Tensor, pos0: int) -> torch.Tensor:
        n, _, d = x.shape
        half = d // 2
        ang = torch.arange(pos0, pos0 + n, dtype=torch.float64, device=x.device)[:, None] * self._inv
        c = ang.cos().float()[:, None, :]
        s = ang.sin().float()[:, None, :]
        x1, x2 = x[..., :half].float(), x[..., half:].float()
        return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1).to(x.dtype)

    def _proj(self, x: torch.Tensor, w: torch.Tensor, heads: int) -> torch.Tensor:
        return (x.to(self.dtype) @ w.to(self.dtype).t()).view(x.shape[0], heads, self.d)

    def _kv(self, x: torch.Tensor, pos0: int):
        k = self._rope(self._proj(x, self.wk, self.hkv), pos0).contiguous()
        v = self._proj(x, self.wv, self.hkv).contiguous()
        return k, v

    def _attend(self, x: torch.Tensor, pos0: int, sel_bufs=None) -> torch.Tensor:
        q = self._rope(self._proj(x, self.wq, self.hq), pos0).contiguous()
        sel = None
        if self.sparse is not None:
            nqp = -(-x.shape[0] // self.page)
            pages, count = sel_bufs if sel_bufs is not None else (
                torch.empty(nqp, self.hkv, self.sparse.stride, dtype=torch.int32, device=self.device),
                torch.empty(nqp, self.hkv, dtype=torch.int32, device=self.device))
            pkv_select_topk_pages(self.pool, 0, pos0, q.detach(), self.sparse.top_k, pages, count,
                                  self.sparse.n_sink, self.sparse.n_local)
            sel = (pages, count)
        o = paged_attention(q, self.pool, 0, pos0, self.scale, sel)
        return x + (o.reshape(x.shape[0], self.hq * self.d) @ self.wo.to(self.dtype).t()).to(x.dtype)

    # ---- the two sweeps
    def forward_sweep(self, xs: List[torch.Tensor]) -> List[torch.Tensor]:
        """No autograd: append every chunk's K/V (chunk order) and return the
        block's outputs.  xs[c]: [n_c][hidden]; chunks are page-aligned."""
        pkv_pool_reset(self.pool, 0)
        pkv_grad_zero(self.pool, 0)
        ys, pos0 = [], 0
        with torch.no_grad():
            for x in xs:
                k, v = self._kv(x, pos0)
                pkv_append_kv(self.pool, 0, pos0, k, v)
                ys.append(self._attend(x, pos0))
                pos0 += x.shape[0]
        return ys

    def backward_sweep(self, xs: List[torch.Tensor], gys: List[torch.Tensor]) -> List[torch.Tensor]:
        """Chunks last to first: recompute the chunk with autograd, back-propagate
        gys[c]; the pool collects dK/dV of every key the chunk attends to; then
        the chunk's own (now complete) dK/dV go back through W_k, W_v.  Adds the
        weight gradients to .grad and returns dL/dx per chunk."""
        starts = [0]
        for x in xs[:-1]:
            starts.append(starts[-1] + x.shape[0])
        dxs: List[Optional[torch.Tensor]] = [None] * len(xs)
        for c in reversed(range(len(xs))):
            pos0, n = starts[c], xs[c].shape[0]
            x = xs[c].detach().requires_grad_()
            y = self._attend(x, pos0)
            torch.autograd.backward(y, gys[c])
            k, v = self._kv(x, pos0)
            dk = torch.empty(n, self.hkv, self.d, dtype=torch.float32, device=self.device)
            dv = torch.empty_like(dk)
            pkv_read_rows(self.pool, 0, PKV_DK, pos0, dk)
            pkv_read_rows(self.pool, 0, PKV_DV, pos0, dv)
            torch.autograd.backward([k, v], [dk.to(k.dtype), dv.to(v.dtype)])
            dxs[c] = x.grad
        return dxs

    def pool_bytes(self) -> int:
        from . import pkv_pool_bytes
        return pkv_pool_bytes(self.pool)[0]

    def close(self) -> None:
        self.pool.close()
