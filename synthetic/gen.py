"""Seeded input generator.

Every tensor is drawn from its own numpy substream keyed by
(seed, config id, layer, chunk, tensor id), so any chunk of any layer can be
regenerated on its own, bit for bit.  Values are drawn in fp32 and, for bf16
workloads, rounded to bf16 with round-to-nearest-even (torch's cast); the
arrays handed out hold those rounded values exactly, so a consumer that
upcasts them to fp64 sees exactly what the GPU stores.

Value laws per workload:
  * Q, K, V ~ N(0, 1); dO ~ N(0, 1) * do_scale.
  * rope_base set: Q and K are rotated (rotate-half convention, inverse
    frequency base**(-2i/d)) at their absolute positions before rounding.
  * planted_frac > 0: round(planted_frac * n_pages) pages per KV head, drawn
    without replacement, get one offset vector u = planted_norm * z / |z|,
    z ~ N(0, I_d), added to every key of that page-head.
  * query_targets > 0 (structured queries): for every query page i and KV
    head g, query_targets planted pages are drawn without replacement from
    the planted pages of head g in [n_sink, i - n_local] (fewer if fewer
    exist), and every query of page i in a head of group g gets
    query_affinity x the sum of their offsets u.  Its scores against those
    pages' keys then rise by about query_affinity x |u|^2 each, so attention
    concentrates on a few earlier pages per query page.
  * page table: per KV head, the first n_pages entries of a seeded
    permutation of the slot indices.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config

_Q, _K, _V, _DO, _TABLE, _PLANT, _TARGET = 1, 2, 3, 4, 5, 6, 7
_BLOCK = 512
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = concurrent.futures.ThreadPoolExecutor(n)
    return _POOL


def _rng(seed: int, cid: int, layer: int, chunk: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cid, layer, chunk, tid]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) -> fp32, via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _rope(x: np.ndarray, pos0: int, base: float) -> np.ndarray:
    """Rotate-half RoPE on x[n][heads][d] at positions pos0 .. pos0+n-1.

    Angles are formed in fp64, the rotation itself in fp32 (torch CPU)."""
    import torch
    n, _, d = x.shape
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(pos0, pos0 + n, dtype=np.float64)[:, None] * inv[None, :]
    c = torch.from_numpy(np.cos(ang).astype(np.float32))[:, None, :]
    s = torch.from_numpy(np.sin(ang).astype(np.float32))[:, None, :]
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    x1, x2 = t[..., :half], t[..., half:]
    out = torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)
    return out.numpy()


@dataclass
class ChunkInputs:
    q_pos0: int
    q: np.ndarray    # [n_q][hq][d] float32 (exact stored values)
    k: np.ndarray    # [n_q][hkv][d]
    v: np.ndarray    # [n_q][hkv][d]
    do: np.ndarray   # [n_q][hq][d]

    @property
    def n_q(self) -> int:
        return self.q.shape[0]


class Workload:
    """Lazily generated inputs of one layer of a config."""

    def __init__(self, cfg: Config, seed: int = 0, layer: int = 0):
        self.cfg = cfg
        self.seed = seed
        self.layer = layer
        self._table: Optional[np.ndarray] = None
        self._planted: Optional[dict] = None

    # -- structure -----------------------------------------------------
    def table(self) -> np.ndarray:
        """int32 [hkv][n_pages]: logical page -> slot."""
        if self._table is None:
            cfg = self.cfg
            t = np.empty((cfg.hkv, cfg.n_pages), dtype=np.int32)
            for g in range(cfg.hkv):
                r = _rng(self.seed, cfg.cid, self.layer, g, _TABLE)
                t[g] = r.permutation(cfg.slots)[: cfg.n_pages]
            self._table = t
        return self._table

    def planted(self) -> dict:
        """{kv head: (pages int64[m], offsets float64[m][d])}."""
        if self._planted is None:
            cfg = self.cfg
            out = {}
            m = int(round(cfg.planted_frac * cfg.n_pages))
            for g in range(cfg.hkv):
                if m == 0:
                    out[g] = (np.zeros(0, np.int64), np.zeros((0, cfg.d)))
                    continue
                r = _rng(self.seed, cfg.cid, self.layer, g, _PLANT)
                pages = np.sort(r.choice(cfg.n_pages, size=m, replace=False))
                z = r.standard_normal((m, cfg.d))
                u = cfg.planted_norm * z / np.linalg.norm(z, axis=1, keepdims=True)
                out[g] = (pages.astype(np.int64), u)
            self._planted = out
        return self._planted

    # -- values ---------------------------------------------------------
    def _draw(self, c: int, tid: int, shape) -> np.ndarray:
        """N(0,1) fp32 of `shape`; rows are drawn in blocks of _BLOCK tokens,
        each from its own substream, on a thread pool."""
        out = np.empty(shape, dtype=np.float32)
        n = shape[0]
        nb = -(-n // _BLOCK)

        def fill(b):
            r = np.random.default_rng(np.random.SeedSequence(
                [self.seed, self.cfg.cid, self.layer, c, tid, b]))
            r.standard_normal(out=out[b * _BLOCK:(b + 1) * _BLOCK], dtype=np.float32)

        if nb == 1:
            fill(0)
        else:
            list(_pool().map(fill, range(nb)))
        return out

    def _finish(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.cfg.dtype == "bf16" else x

    def chunk(self, c: int) -> ChunkInputs:
        cfg = self.cfg
        pos0, n = cfg.chunk_range(c)
        q = self._draw(c, _Q, (n, cfg.hq, cfg.d))
        k = self._draw(c, _K, (n, cfg.hkv, cfg.d))
        v = self._draw(c, _V, (n, cfg.hkv, cfg.d))
        do = self._draw(c, _DO, (n, cfg.hq, cfg.d))
        if cfg.do_scale != 1.0:
            do *= np.float32(cfg.do_scale)
        if cfg.planted_frac > 0:
            k = k.astype(np.float64)
            for g, (pages, u) in self.planted().items():
                for p, off in zip(pages, u):
                    lo = max(int(p) * cfg.page, pos0)
                    hi = min((int(p) + 1) * cfg.page, pos0 + n)
                    if lo < hi:
                        k[lo - pos0:hi - pos0, g, :] += off
            k = k.astype(np.float32)
        if cfg.query_targets > 0:
            q = q.astype(np.float64)
            G = cfg.hq // cfg.hkv
            for i in range(pos0 // cfg.page, (pos0 + n - 1) // cfg.page + 1):
                lo, hi = max(i * cfg.page, pos0) - pos0, min((i + 1) * cfg.page, pos0 + n) - pos0
                for g, (pages, u) in self.planted().items():
                    ok = np.nonzero((pages >= cfg.n_sink) & (pages <= i - cfg.n_local))[0]
                    if ok.size == 0:
                        continue
                    r = np.random.default_rng(np.random.SeedSequence(
                        [self.seed, cfg.cid, self.layer, i, _TARGET, g]))
                    pick = r.choice(ok, size=min(cfg.query_targets, ok.size), replace=False)
                    q[lo:hi, g * G:(g + 1) * G, :] += cfg.query_affinity * u[pick].sum(axis=0)
            q = q.astype(np.float32)
        if cfg.rope_base:
            q = _rope(q, pos0, cfg.rope_base)
            k = _rope(k, pos0, cfg.rope_base)
        return ChunkInputs(pos0, self._finish(q), self._finish(k),
                           self._finish(v), self._finish(do))

    def full(self) -> ChunkInputs:
        """All chunks concatenated (q_pos0 = 0); for small contexts."""
        parts = [self.chunk(c) for c in range(self.cfg.n_chunks)]
        return ChunkInputs(0, *(np.concatenate([getattr(p, f) for p in parts])
                                for f in ("q", "k", "v", "do")))

    def keys(self, upto: int) -> tuple[np.ndarray, np.ndarray]:
        """K, V of tokens [0, upto) (concatenating chunks)."""
        ks, vs = [], []
        for c in range(self.cfg.n_chunks):
            pos0, n = self.cfg.chunk_range(c)
            if pos0 >= upto:
                break
            ch = self.chunk(c)
            m = min(n, upto - pos0)
            ks.append(ch.k[:m])
            vs.append(ch.v[:m])
        return np.concatenate(ks), np.concatenate(vs)
