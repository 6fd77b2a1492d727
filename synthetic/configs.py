"""Workload shapes.

The attention shape is the Qwen2.5-7B one the OOMB summaries evaluate on
(gist.science OOMB summaries, "Results" sections): 28 query heads, 4 KV heads,
head_dim 128.  The pages fix no page size, chunk size, top-K budget or data
type; the values below are the ones this library is measured at, written out
with their sizes.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    n_ctx: int            # tokens in the whole context
    chunk: int            # query-chunk length; the last chunk may be shorter
    page: int             # tokens per KV page
    hq: int               # query heads
    hkv: int              # KV heads
    d: int                # head dim
    dtype: str            # "f32" or "bf16" (storage); accumulation is fp32
    slots: int            # HBM page slots per layer per KV head
    table: str            # "injection" (pages scattered into a larger slot pool) or "permutation"
    sparse: bool = False
    top_k: int = 0
    n_sink: int = 1
    n_local: int = 2
    rope_base: Optional[float] = None
    do_scale: float = 1.0
    planted_frac: float = 0.0
    planted_norm: float = 0.0
    # structured queries (optional): each query page is drawn toward
    # `query_targets` planted key pages among its candidates, its queries
    # getting query_affinity x the sum of those pages' offsets (per KV group),
    # so that attention concentrates on a few pages per query page
    query_targets: int = 0
    query_affinity: float = 0.0
    host_tier: bool = False
    hbm_cap_bytes: int = 0
    cid: int = 0          # stream id used to key the seeded substreams

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def n_pages(self) -> int:
        return -(-self.n_ctx // self.page)

    @property
    def n_chunks(self) -> int:
        return -(-self.n_ctx // self.chunk)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def chunk_range(self, c: int) -> tuple[int, int]:
        lo = c * self.chunk
        return lo, min(self.chunk, self.n_ctx - lo)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


QWEN = dict(hq=28, hkv=4, d=128)

CONFIGS = {
    # Tiny fp32, dense: 512 tokens, 4 chunks of 128, pages of 16, GQA 2:1, d 64,
    # 40 slots holding the 32 logical pages at seeded positions.
    "tiny_f32": Config("tiny_f32", 1, 512, 128, 16, 2, 1, 64, "f32", 40,
                       "injection", cid=0),
    # Qwen shape, 32K dense, 8 chunks of 4096, pages of 128, RoPE base 1e6.
    "qwen_32k_dense": Config("qwen_32k_dense", 1, 32768, 4096, 128, dtype="bf16",
                             slots=256, table="permutation", rope_base=1e6,
                             do_scale=1.0 / 64.0, cid=1, **QWEN),
    # Qwen shape, 128K dense, chunks of 12288 (10 full + one of 8192).
    "qwen_128k_dense": Config("qwen_128k_dense", 1, 131072, 12288, 128, dtype="bf16",
                              slots=1024, table="permutation", rope_base=1e6,
                              do_scale=1.0 / 64.0, cid=2, **QWEN),
    # Qwen shape, 256K page top-K (K=64 + page 0 + 2 most recent), chunks of 4096,
    # keys with a planted offset of norm 2 on 5% of page-heads.
    "qwen_256k_topk": Config("qwen_256k_topk", 1, 262144, 4096, 128, dtype="bf16",
                             slots=2048, table="permutation", sparse=True, top_k=64,
                             planted_frac=0.05, planted_norm=2.0, cid=3, **QWEN),
    # 28 layers of the 128K dense workload with every layer's pools in pinned host
    # memory and a 16 GiB HBM cap (the dense offloaded stack).
    "qwen_128k_dense_offload": Config("qwen_128k_dense_offload", 28, 131072, 12288, 128,
                                      dtype="bf16", slots=1024, table="permutation",
                                      rope_base=1e6, do_scale=1.0 / 64.0, host_tier=True,
                                      hbm_cap_bytes=16 << 30, cid=5, **QWEN),
    # 28 layers, 1M tokens, top-K 128, pools in pinned host memory, 16 GiB HBM cap.
    "qwen_1m_offload": Config("qwen_1m_offload", 28, 1048576, 8192, 128, dtype="bf16",
                              slots=8192, table="permutation", sparse=True, top_k=128,
                              planted_frac=0.05, planted_norm=2.0, host_tier=True,
                              hbm_cap_bytes=16 << 30, cid=4, **QWEN),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def mini_config(base: str, n_ctx: int, chunk: int, slots: Optional[int] = None,
                **kw) -> Config:
    """A reduced-context copy of a named config with the same head shape and
    value laws (for tests the oracle finishes in seconds)."""
    cfg = CONFIGS[base]
    pages = -(-n_ctx // cfg.page)
    if slots is None:
        slots = pages + (8 if cfg.table == "injection" else 0)
    return cfg.replace(name=f"{base}@{n_ctx}", n_ctx=n_ctx, chunk=chunk,
                       slots=slots, **kw)
