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

from . import (PKV_BF16, PKV_F32, Pool, pkv_append_kv, pkv_attn_bwd, pkv_attn_fwd,
               pkv_select_topk_pages)


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
        self.sel = None
        if sparse is not None:
            nqp = -(-n_q // page)
            self.sel = (torch.empty(nqp, hkv, sparse.stride, dtype=torch.int32, device=device),
                        torch.empty(nqp, hkv, dtype=torch.int32, device=device))


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
