"""Seeded inputs drawn on the GPU (torch's device generator), for the
full-size workloads whose CPU generation would take minutes.

Same value laws, page tables and planted pages as synthetic.gen.Workload
(the tables and planted offsets are taken from it), but the Gaussian draws
come from torch's device generator, seeded per (seed, config id, layer,
chunk, tensor id); the values therefore differ from the CPU generator's.
Anything that needs them on the host (the oracle's sampled checks) copies
the generated tensors back.  No attention arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Config
from .gen import Workload, _DO, _K, _Q, _V


def _seed(*key) -> int:
    return int(np.random.SeedSequence(list(key)).generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


class GpuWorkload:
    def __init__(self, cfg: Config, seed: int = 0, layer: int = 0, device: str = "cuda"):
        self.cfg = cfg
        self.seed = seed
        self.layer = layer
        self.device = device
        self.cpu = Workload(cfg, seed, layer)
        self._rope_inv = None
        self._planted = None

    def table(self) -> np.ndarray:
        return self.cpu.table()

    @property
    def dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32

    def _draw(self, c: int, tid: int, shape) -> torch.Tensor:
        g = torch.Generator(device=self.device)
        g.manual_seed(_seed(self.seed, 1000 + self.cfg.cid, self.layer, c, tid))
        return torch.randn(shape, generator=g, device=self.device, dtype=torch.float32)

    def _rope(self, x: torch.Tensor, pos0: int) -> torch.Tensor:
        # angles computed on the device (fp64): no host-to-device copy, which
        # from pageable memory would synchronise the host with the device
        # (and, on the default stream, with every other stream) in the middle
        # of a timed sweep
        n, _, d = x.shape
        half = d // 2
        dev = x.device
        inv = float(self.cfg.rope_base) ** (
            -torch.arange(half, dtype=torch.float64, device=dev) * 2.0 / d)
        ang = torch.arange(pos0, pos0 + n, dtype=torch.float64, device=dev)[:, None] * inv[None, :]
        c = torch.cos(ang).to(torch.float32)[:, None, :]
        s = torch.sin(ang).to(torch.float32)[:, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)

    def chunk(self, c: int, parts: str = "qkvd") -> dict:
        """{'q_pos0', 'q', 'k', 'v', 'do'} as device tensors in the storage
        dtype; `parts` limits which tensors are drawn (each has its own
        substream, so a subset gives the same values)."""
        cfg = self.cfg
        pos0, n = cfg.chunk_range(c)
        out = dict(q_pos0=pos0)
        dt = self.dtype
        if "q" in parts:
            q = self._draw(c, _Q, (n, cfg.hq, cfg.d))
            if cfg.rope_base:
                q = self._rope(q, pos0)
            out["q"] = q.to(dt).contiguous()
        if "d" in parts:
            do = self._draw(c, _DO, (n, cfg.hq, cfg.d))
            if cfg.do_scale != 1.0:
                do *= cfg.do_scale
            out["do"] = do.to(dt).contiguous()
        if "v" in parts:
            out["v"] = self._draw(c, _V, (n, cfg.hkv, cfg.d)).to(dt).contiguous()
        if "k" in parts:
            out["k"] = self._keys(c, pos0, n).to(dt).contiguous()
        return out

    def _keys(self, c: int, pos0: int, n: int) -> torch.Tensor:
        cfg = self.cfg
        k = self._draw(c, _K, (n, cfg.hkv, cfg.d))
        if cfg.planted_frac > 0:
            for g, (pages, u) in self.cpu.planted().items():
                lo_p, hi_p = pos0 // cfg.page, (pos0 + n - 1) // cfg.page
                sel = (pages >= lo_p) & (pages <= hi_p)
                for p, off in zip(pages[sel], u[sel]):
                    lo = max(int(p) * cfg.page, pos0)
                    hi = min((int(p) + 1) * cfg.page, pos0 + n)
                    k[lo - pos0:hi - pos0, g, :] += torch.from_numpy(off.astype(np.float32)).to(self.device)
        if cfg.rope_base:
            k = self._rope(k, pos0)
        return k
