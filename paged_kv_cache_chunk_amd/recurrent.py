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
                 seed: int = 0, device: str = "cuda", pool=None, layer: int = 0):
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
        # a block of its own, or layer `layer` of a pool shared by a stack
        self.own_pool = pool is None
        self.pool = pkv_pool_create(1, hkv, d, page, pages, pages, kvd) if pool is None else pool
        self.layer = layer
        # selection of each chunk (by its first position), kept from the
        # forward sweep for the backward sweep: the selection is a constant of
        # the gradient and recomputing it from the same queries gives the same
        self.sels = {}
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

    def _q(self, x: torch.Tensor, pos0: int) -> torch.Tensor:
        return self._rope(self._proj(x, self.wq, self.hq), pos0).contiguous()

    def select(self, q: torch.Tensor, pos0: int):
        """Top-K selection of the chunk at pos0 (kept in self.sels); None in
        dense mode."""
        if self.sparse is None:
            return None
        nqp = -(-q.shape[0] // self.page)
        pages = torch.empty(nqp, self.hkv, self.sparse.stride, dtype=torch.int32, device=self.device)
        count = torch.empty(nqp, self.hkv, dtype=torch.int32, device=self.device)
        pkv_select_topk_pages(self.pool, self.layer, pos0, q.detach(), self.sparse.top_k, pages,
                              count, self.sparse.n_sink, self.sparse.n_local)
        self.sels[pos0] = (pages, count)
        return self.sels[pos0]

    def _out(self, x: torch.Tensor, o: torch.Tensor) -> torch.Tensor:
        return x + (o.reshape(x.shape[0], self.hq * self.d) @ self.wo.to(self.dtype).t()).to(x.dtype)

    def _attend(self, x: torch.Tensor, pos0: int, q: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The block on one chunk; the selection is the one kept for pos0 (made
        here if there is none)."""
        if q is None:
            q = self._q(x, pos0)
        sel = None
        if self.sparse is not None:
            sel = self.sels.get(pos0) or self.select(q, pos0)
        o = paged_attention(q, self.pool, self.layer, pos0, self.scale, sel)
        return self._out(x, o)

    # ---- the two sweeps
    def forward_sweep(self, xs: List[torch.Tensor]) -> List[torch.Tensor]:
        """No autograd: append every chunk's K/V (chunk order) and return the
        block's outputs.  xs[c]: [n_c][hidden]; chunks are page-aligned."""
        pkv_pool_reset(self.pool, self.layer)
        pkv_grad_zero(self.pool, self.layer)
        self.sels = {}
        ys, pos0 = [], 0
        with torch.no_grad():
            for x in xs:
                k, v = self._kv(x, pos0)
                pkv_append_kv(self.pool, self.layer, pos0, k, v)
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
            pkv_read_rows(self.pool, self.layer, PKV_DK, pos0, dk)
            pkv_read_rows(self.pool, self.layer, PKV_DV, pos0, dv)
            torch.autograd.backward([k, v], [dk.to(k.dtype), dv.to(v.dtype)])
            dxs[c] = x.grad
        return dxs

    def pool_bytes(self) -> int:
        from . import pkv_pool_bytes
        return pkv_pool_bytes(self.pool)[0]

    def close(self) -> None:
        if self.own_pool:
            self.pool.close()


class AttentionStack:
    """n_layers attention blocks (x_{l+1} = x_l + W_o attn(...)) trained
    chunk-recurrently over one n_layers-layer pool, optionally with every
    layer's K/V and KV gradients in pinned host memory ("Out of the Memory
    Barrier", gist.science de, sections 2.A-2.D; sciencestack.ai, Figure 3).

    Forward sweep (no autograd), chunk by chunk, layer by layer: project,
    append the chunk's K/V, select (top-K), attend.  Backward sweep, chunks
    last to first: the chunk's forward is recomputed layer by layer (only
    the chunk's layer inputs are kept), then the layers run backward top to
    bottom with autograd; the attention backward adds dK/dV into the layer's
    gradient pages and the chunk's own completed dK/dV go back through W_k,
    W_v.  The selections of the forward sweep are kept for both passes.

    With host_tier, a side stream fetches each layer's pages (dense: every
    key up to the chunk's end; top-K: the selected pages) into one of two HBM
    windows one layer ahead, while the current layer's projections and
    attention run (de 2.C: prefetch of the next layer; with sparse attention
    the transfer overlaps the K/V projections); the backward's fetches bring
    the pages' accumulated gradients, and a third stream writes each layer's
    gradient pages back after its backward.  With host_grad_accumulate the
    backward's fetches bring K/V only: the window's gradients start at zero,
    the writeback sends the visit's contributions, and the library's host
    threads add them into the host tier (the chunk's own dK/dV rows are then
    read as window plus tier).  In the forward sweep of a dense
    stack the next layer's prefix is fetched before its chunk is appended
    (the append then writes the window too); in top-K mode a layer's
    selection needs its chunk's page representatives, so its fetch waits for
    its own append and selection.
    """

    def __init__(self, n_layers: int, hidden: int = 3584, hq: int = 28, hkv: int = 4,
                 d: int = 128, rope_base: float = 1e6, page: int = 128,
                 max_tokens: int = 131072, sparse: Optional[Sparse] = None,
                 dtype: torch.dtype = torch.bfloat16, seed: int = 0, device: str = "cuda",
                 host_tier: bool = False, host_grad_dtype: int = PKV_F32,
                 window_slots: int = 0, host_grad_accumulate: bool = False):
        pages = -(-max_tokens // page)
        kvd = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
        self.pool = pkv_pool_create(n_layers, hkv, d, page, pages, pages, kvd,
                                    host_tier=int(host_tier), host_grad_dtype=host_grad_dtype,
                                    window_slots=window_slots if host_tier else 0,
                                    host_grad_accumulate=int(host_tier and host_grad_accumulate))
        self.blocks = [AttentionBlock(hidden, hq, hkv, d, rope_base, page, max_tokens, sparse,
                                      dtype, seed + l, device, pool=self.pool, layer=l)
                       for l in range(n_layers)]
        self.L, self.page, self.sparse, self.host_tier = n_layers, page, sparse, host_tier
        self.hkv, self.d, self.device = hkv, d, device
        self.copy = torch.cuda.Stream() if host_tier else None
        self.wb = torch.cuda.Stream() if host_tier else None

    def parameters(self) -> List[torch.Tensor]:
        return [w for b in self.blocks for w in b.parameters()]

    # ---- host tier: the fetch of one layer's pages for one chunk
    def _fetch(self, l: int, pos0: int, n: int, with_grads: bool) -> None:
        """On the copy stream, after the work enqueued so far on the current
        stream: dense, the pages of keys 0 .. pos0 + n - 1; top-K, the pages
        of the chunk's selection (made already)."""
        if not self.host_tier:
            return
        from . import pkv_prefetch_pages, pkv_prefetch_prefix
        ev = torch.cuda.Event()
        ev.record()
        self.copy.wait_event(ev)
        if self.sparse is None:
            pkv_prefetch_prefix(self.pool, l, pos0 + n, with_grads=with_grads, copy_stream=self.copy)
        else:
            pkv_prefetch_pages(self.pool, l, self.blocks[l].sels[pos0], with_grads=with_grads,
                               copy_stream=self.copy)

    def _writeback(self, l: int) -> None:
        if self.host_tier:
            from . import pkv_writeback_grads
            pkv_writeback_grads(self.pool, l, copy_stream=self.wb)

    # ---- the two sweeps
    def forward_sweep(self, xs: List[torch.Tensor]) -> List[torch.Tensor]:
        """No autograd; returns the top layer's outputs per chunk."""
        for b in self.blocks:
            pkv_pool_reset(self.pool, b.layer)
            pkv_grad_zero(self.pool, b.layer)
            b.sels = {}
        ys, pos0 = [], 0
        dense_ahead = self.host_tier and self.sparse is None
        with torch.no_grad():
            for x in xs:
                n = x.shape[0]
                if dense_ahead:
                    self._fetch(0, pos0, n, False)
                for l, b in enumerate(self.blocks):
                    if dense_ahead and l + 1 < self.L:
                        self._fetch(l + 1, pos0, n, False)  # ahead of its append
                    q = b._q(x, pos0)
                    k, v = b._kv(x, pos0)
                    pkv_append_kv(self.pool, l, pos0, k, v)
                    if self.sparse is not None:
                        b.select(q, pos0)
                        self._fetch(l, pos0, n, False)
                    x = b._attend(x, pos0, q)
                ys.append(x)
                pos0 += n
        return ys

    def backward_sweep(self, xs: List[torch.Tensor], gys: List[torch.Tensor]) -> List[torch.Tensor]:
        """Chunks last to first; adds the weight gradients to .grad and returns
        dL/dx of the stack's input per chunk."""
        L = self.L
        starts = [0]
        for x in xs[:-1]:
            starts.append(starts[-1] + x.shape[0])
        dxs: List[Optional[torch.Tensor]] = [None] * len(xs)
        for c in reversed(range(len(xs))):
            pos0, n = starts[c], xs[c].shape[0]
            # 1. recompute the chunk's forward, keeping each layer's input; the
            #    top layer's fetch brings its gradients too (its backward is next)
            acts = []
            x = xs[c]
            self._fetch(0, pos0, n, L == 1)
            with torch.no_grad():
                for l, b in enumerate(self.blocks):
                    if l + 1 < L:
                        self._fetch(l + 1, pos0, n, l + 1 == L - 1)
                    acts.append(x)
                    x = b._attend(x, pos0)
            # 2. backward, top to bottom, the next layer down fetched one ahead
            gy = gys[c]
            for l in reversed(range(L)):
                b = self.blocks[l]
                if l - 1 >= 0:
                    self._fetch(l - 1, pos0, n, True)
                xl = acts[l].detach().requires_grad_()
                y = b._attend(xl, pos0)
                torch.autograd.backward(y, gy)
                k, v = b._kv(xl, pos0)
                dk = torch.empty(n, self.hkv, self.d, dtype=torch.float32, device=self.device)
                dv = torch.empty_like(dk)
                pkv_read_rows(self.pool, l, PKV_DK, pos0, dk)
                pkv_read_rows(self.pool, l, PKV_DV, pos0, dv)
                torch.autograd.backward([k, v], [dk.to(k.dtype), dv.to(v.dtype)])
                self._writeback(l)
                gy = xl.grad
            dxs[c] = gy
        return dxs

    def pool_bytes(self) -> tuple:
        from . import pkv_pool_bytes
        return pkv_pool_bytes(self.pool)

    def close(self) -> None:
        torch.cuda.synchronize()
        self.pool.close()
