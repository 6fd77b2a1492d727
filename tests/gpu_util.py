"""Helpers for GPU tests: run a workload through libpkv and compare with the
oracle (the oracle is imported by the tests, not here)."""
from __future__ import annotations

import numpy as np

from synthetic import Workload


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def run_layer(cfg, w: Workload, sparse=None, table=None, order="reverse", chunks=None):
    """Append every chunk of one layer, then run select (sparse) + fwd + bwd per
    chunk (in reverse chunk order by default, as a backward sweep does).
    Returns dict O [N][hq][d], lse [hq][N], dq, dk, dv [N][hkv][d] (numpy
    float64), sel (per chunk: (pages, count) numpy) and the chunk inputs."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, chunk_step, torch_dtype

    kvd = pkv.PKV_BF16 if cfg.dtype == "bf16" else pkv.PKV_F32
    dt = torch_dtype(kvd)
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, kvd)
    tab = w.table() if table is None else table
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    if chunks is None:
        chunks = [w.chunk(c) for c in range(cfg.n_chunks)]
    for ch in chunks:
        k = torch.from_numpy(ch.k).to(dt).cuda()
        v = torch.from_numpy(ch.v).to(dt).cuda()
        pkv.pkv_append_kv(pool, 0, ch.q_pos0, k, v)
    N = cfg.n_ctx
    O = np.zeros((N, cfg.hq, cfg.d))
    lse = np.zeros((cfg.hq, N))
    dq = np.zeros((N, cfg.hq, cfg.d))
    sels = [None] * len(chunks)
    idx = range(len(chunks))
    if order == "reverse":
        idx = reversed(list(idx))
    for c in idx:
        ch = chunks[c]
        n = ch.n_q
        buf = ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page, dt, sparse)
        q = torch.from_numpy(ch.q).to(dt).cuda()
        do = torch.from_numpy(ch.do).to(dt).cuda()
        chunk_step(pool, 0, ch.q_pos0, q, do, buf.o, buf.lse, buf.dq, cfg.scale, sparse,
                   buf.sel)
        torch.cuda.synchronize()
        sl = slice(ch.q_pos0, ch.q_pos0 + n)
        O[sl] = buf.o.float().cpu().numpy()
        lse[:, sl] = buf.lse.cpu().numpy()
        dq[sl] = buf.dq.cpu().numpy()
        if sparse is not None:
            sels[c] = (buf.sel[0].cpu().numpy(), buf.sel[1].cpu().numpy())
    dk = torch.empty(N, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dv)
    torch.cuda.synchronize()
    out = dict(O=O, lse=lse, dq=dq, dk=dk.cpu().numpy().astype(np.float64),
               dv=dv.cpu().numpy().astype(np.float64), sel=sels, chunks=chunks, pool=pool)
    return out


def sel_lists(sel_np):
    """(pages [nqp][hkv][stride], count [nqp][hkv]) -> nested python lists."""
    pages, count = sel_np
    return [[list(map(int, pages[i, g, :count[i, g]])) for g in range(pages.shape[1])]
            for i in range(pages.shape[0])]


def compare_selection(gpu_sel, ref_sel, ref_scores, top_k, gap=1e-5):
    """Selections must be equal except for candidates within `gap` of the
    K-th score.  Returns the number of (query page, head) lists that differ."""
    n_diff = 0
    for i, (row_g, row_r) in enumerate(zip(gpu_sel, ref_sel)):
        for g, (a, b) in enumerate(zip(row_g, row_r)):
            a, b = set(a), set(map(int, b))
            if a == b:
                continue
            n_diff += 1
            cand, s = ref_scores[(i, g)]
            kth = np.sort(s)[::-1][min(top_k, len(s)) - 1]
            for j in a ^ b:
                assert j in set(cand.tolist()), f"forced page {j} differs (page {i}, head {g})"
                sj = s[list(cand).index(j)]
                assert abs(sj - kth) < gap, f"page {j} off by {abs(sj - kth)} (page {i}, head {g})"
    return n_diff
