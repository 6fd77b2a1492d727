"""Chunk-recurrent driver over libpkv (host-side orchestration only).

The sequence is processed in query chunks ("Out of the Memory Barrier",
gist.science de, section 2.A): each chunk's K/V are appended to the paged
cache, then the chunk's attention runs over every earlier page plus its own
causal part; the backward recomputes from the saved log-sum-exp and adds the
chunk's dK/dV into the paged gradient pool.  Every step is a libpkv call.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import PKV_BF16, Pool, pkv_attn_bwd, pkv_attn_fwd, pkv_select_topk_pages


def torch_dtype(kv_dtype: int) -> torch.dtype:
    return torch.bfloat16 if kv_dtype == PKV_BF16 else torch.float32


@dataclass
class Sparse:
    top_k: int
    n_sink: int = 1
    n_local: int = 2

    @property
    def stride(self) -> int:
        return self.top_k + self.n_sink + self.n_local


class ChunkBuffers:
    """Device buffers of one query chunk (allocated once, reused)."""

    def __init__(self, n_q: int, hq: int, hkv: int, d: int, page: int, dtype: torch.dtype,
                 sparse: Optional[Sparse], device="cuda"):
        self.o = torch.empty(n_q, hq, d, dtype=dtype, device=device)
        self.lse = torch.empty(hq, n_q, dtype=torch.float32, device=device)
        self.dq = torch.empty(n_q, hq, d, dtype=torch.float32, device=device)
        self.sel = self.own_sel = None  # sel: the selection in use (own_sel or one kept elsewhere)
        if sparse is not None:
            nqp = -(-n_q // page)
            self.own_sel = (torch.empty(nqp, hkv, sparse.stride, dtype=torch.int32, device=device),
                            torch.empty(nqp, hkv, dtype=torch.int32, device=device))
            self.sel = self.own_sel


def chunk_step(pool: Pool, layer: int, q_pos0: int, q, do, o, lse, dq, scale: float,
               sparse: Optional[Sparse] = None, sel=None, forward: bool = True,
               stream=None):
    """One chunk: (select) + forward + recompute-backward, all on `stream`."""
    if sparse is not None:
        pkv_select_topk_pages(pool, layer, q_pos0, q, sparse.top_k, sel[0], sel[1],
                              sparse.n_sink, sparse.n_local, stream=stream)
    if forward:
        pkv_attn_fwd(pool, layer, q_pos0, q, o, lse, scale, sel=sel, stream=stream)
    pkv_attn_bwd(pool, layer, q_pos0, q, o, do, lse, dq, scale, sel=sel, stream=stream)


class OffloadSweep:
    """Backward sweep of a stack of attention layers whose KV pools live in a
    host tier ("Out of the Memory Barrier", gist.science de, section 2.C: the
    next layer's KV is fetched while the current layer computes; the KV
    gradients travel the same way; section 2.D: with page top-K only the
    selected pages move).

    For each chunk (last to first) and each layer (last to first): the
    layer's selection is computed on the compute stream one layer ahead, its
    pages (and their gradients) are prefetched on the copy stream while the
    current layer's forward + backward run, and each layer's gradient pages
    are written back on a third stream after its backward.  Only events
    order the streams; the host never waits on the device inside the sweep,
    except that with host_grad_accumulate a writeback first waits until the
    host adds of its window's previous writeback have freed the staging.

    inputs(layer, chunk) -> dict(q_pos0, q, do) of device tensors.

    sels: optional {(layer, chunk): (pages, count)} made beforehand, e.g. by
    the forward sweep (select_all): the backward sweep then reuses them (the
    selection is a constant of the gradient) instead of selecting again
    beside the copy kernels, whose host reads slow small kernels down.
    """

    def __init__(self, pool: Pool, n_layers: int, hq: int, hkv: int, d: int, page: int,
                 scale: float, sparse: Optional[Sparse], dtype: torch.dtype,
                 compute_stream=None, copy_stream=None, writeback_stream=None, sels=None):
        self.pool, self.L, self.hq, self.hkv, self.d, self.page = pool, n_layers, hq, hkv, d, page
        self.scale, self.sparse, self.dtype = scale, sparse, dtype
        self.compute = compute_stream or torch.cuda.current_stream()
        # host -> HBM fetches and HBM -> host writebacks on separate streams so
        # that both directions of the host link are busy at once
        self.copy = copy_stream or torch.cuda.Stream()
        self.wb = writeback_stream or torch.cuda.Stream()
        self.sels = sels

    def select_all(self, layers, chunks, inputs) -> dict:
        """Selections of the given (layer, chunk) pairs, on the compute stream
        (what a forward sweep computes and the backward sweep reuses); kept in
        self.sels and returned."""
        out = {} if self.sels is None else self.sels
        if self.sparse is None:
            return out
        for c in chunks:
            for layer in layers:
                ch = inputs(layer, c)
                nqp = -(-ch["q"].shape[0] // self.page)
                pages = torch.empty(nqp, self.hkv, self.sparse.stride, dtype=torch.int32,
                                    device=ch["q"].device)
                count = torch.empty(nqp, self.hkv, dtype=torch.int32, device=ch["q"].device)
                pkv_select_topk_pages(self.pool, layer, ch["q_pos0"], ch["q"], self.sparse.top_k,
                                      pages, count, self.sparse.n_sink, self.sparse.n_local,
                                      stream=self.compute)
                out[(layer, ch["q_pos0"])] = (pages, count)
        self.sels = out
        return out

    def _select(self, layer: int, ch: dict, buf: ChunkBuffers):
        if self.sparse is None:
            return None
        if self.sels and (layer, ch["q_pos0"]) in self.sels:
            buf.sel = self.sels[(layer, ch["q_pos0"])]
            return buf.sel
        sel = buf.sel = buf.own_sel
        pkv_select_topk_pages(self.pool, layer, ch["q_pos0"], ch["q"], self.sparse.top_k,
                              sel[0], sel[1], self.sparse.n_sink, self.sparse.n_local,
                              stream=self.compute)
        return sel

    def _prefetch(self, layer: int, ch: dict, sel):
        """The layer's pages for this chunk, with their gradients: the
        selected pages (top-K), or the pages of keys 0 .. the chunk's last
        query (dense; later pages are neither read nor changed)."""
        from . import pkv_prefetch_pages, pkv_prefetch_prefix
        if sel is None:
            pkv_prefetch_prefix(self.pool, layer, ch["q_pos0"] + ch["q"].shape[0], with_grads=True,
                                copy_stream=self.copy)
        else:
            pkv_prefetch_pages(self.pool, layer, sel, with_grads=True, copy_stream=self.copy)

    def _select_and_prefetch(self, layer: int, ch: dict, buf):
        sel = self._select(layer, ch, buf)
        ev = torch.cuda.Event()
        ev.record(self.compute)
        self.copy.wait_event(ev)
        self._prefetch(layer, ch, sel)
        return sel

    def chunk(self, c: int, inputs, bufs, outputs=None, next_chunk=None):
        """Backward-sweep step of chunk c over every layer.  bufs[layer]:
        ChunkBuffers sized for this chunk (two alternating sets suffice).
        outputs(layer, c, buf) is called after the layer's backward is
        enqueued (on the compute stream) to collect results.

        next_chunk = (c_next, bufs_next): the chunk the caller runs next and
        its buffers.  While layer 0 of chunk c computes, the top layer of
        c_next is selected and prefetched, so that the next call does not
        start with a fetch that nothing overlaps (only when the two layers
        use different windows, i.e. an even number of layers)."""
        from . import pkv_writeback_grads
        L = self.L
        ahead = getattr(self, "_ahead", None)
        self._ahead = None
        sels = {}
        if ahead is not None and ahead[0] == c:
            ins = {L - 1: ahead[1]}
            sels[L - 1] = ahead[2]
        else:
            ins = {L - 1: inputs(L - 1, c)}
            sels[L - 1] = self._select_and_prefetch(L - 1, ins[L - 1], bufs[L - 1])
        for layer in range(L - 1, -1, -1):
            if layer - 1 >= 0:
                ins[layer - 1] = inputs(layer - 1, c)
                sels[layer - 1] = self._select_and_prefetch(layer - 1, ins[layer - 1],
                                                            bufs[layer - 1])
            elif next_chunk is not None and L % 2 == 0:
                c_next, bufs_next = next_chunk
                ch_next = inputs(L - 1, c_next)
                sel_next = self._select_and_prefetch(L - 1, ch_next, bufs_next[L - 1])
                self._ahead = (c_next, ch_next, sel_next)
            ch, b, sel = ins.pop(layer), bufs[layer], sels.pop(layer)
            pkv_attn_fwd(self.pool, layer, ch["q_pos0"], ch["q"], b.o, b.lse, self.scale,
                         sel=sel, stream=self.compute)
            pkv_attn_bwd(self.pool, layer, ch["q_pos0"], ch["q"], b.o, ch["do"], b.lse, b.dq,
                         self.scale, sel=sel, stream=self.compute)
            if outputs is not None:
                outputs(layer, c, b)
            pkv_writeback_grads(self.pool, layer, copy_stream=self.wb)
