#!/usr/bin/env python3
"""Benchmark of the paged-KV chunk attention hot path on one MI355X.

One step = one attention layer over the whole context, chunk by chunk, as a
chunk-recurrent training step runs it: the layer's pool is reset and every
chunk's K/V appended (forward sweep), then, in reverse chunk order (backward
sweep), each chunk runs (page selection in top-K mode) + attention forward +
recompute-backward, the backward adding dK/dV into the paged gradient pool.
Inputs (seeded, synthetic, Qwen2.5-7B attention shape) are resident in HBM
before the timed region.

Headline: 128K-token dense context (chunks of 12288, pages of 128); the
256K-token page top-K context (top-K 64 + page 0 + 2 local pages, chunks of
4096) is reported in the same line.  FLOPs use the algorithmic count
14 * d * Hq per attended (query, key) pair (4 d forward + 10 d backward).

Prints ONE JSON line.  --gpus N with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# x d x Hq per attended (query, key) pair.  Executed: what each kernel
# computes (the dQ kernel recomputes S and dP, so the three kernels execute
# 18 d per pair); algorithmic: the kernel's share of the 14 d a training step
# needs (forward 4 d; backward 10 d = S 2 + dP 2 + dV 2 + dK 2 in the dK/dV
# kernel, dQ 2 in the dQ kernel).
KERNEL_FLOPS_PER_PAIR = {"fwd": 4, "dq": 6, "dkdv": 8}
KERNEL_FLOPS_ALGORITHMIC = {"fwd": 4, "dq": 2, "dkdv": 8}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the bf16 attention and measurement kernel sources and their
    compile flags: stored counter readings only apply to the kernels they were
    taken on."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "paged_kv_cache_chunk_amd")
    for p in sorted(glob.glob(os.path.join(pkg, "csrc", "attn_bf16_*"))) + [
            os.path.join(pkg, "csrc", "micro.hip"), os.path.join(pkg, "build.py")]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def sparse_pairs(sel_counts, chunk_rows, page: int, G: int) -> int:
    """Attended (query, key) pairs x heads from the selection counts of one chunk.
    Every listed page before the query page is complete; the query page itself
    contributes its causal triangle."""
    total = 0
    nqp, hkv = sel_counts.shape
    for i in range(nqp):
        rows = min(page, chunk_rows - i * page)
        for g in range(hkv):
            c = int(sel_counts[i, g])
            total += G * ((c - 1) * page * rows + rows * (rows + 1) // 2)
    return total


class LayerBench:
    """Inputs, pool and buffers of one single-layer workload."""

    def __init__(self, cfg, seed: int = 0):
        import torch
        import paged_kv_cache_chunk_amd as pkv
        from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, Sparse
        from synthetic.gpu import GpuWorkload

        self.cfg = cfg
        self.pkv = pkv
        self.w = GpuWorkload(cfg, seed=seed)
        t0 = time.time()
        self.chunks = [self.w.chunk(c) for c in range(cfg.n_chunks)]
        torch.cuda.synchronize()
        log(f"[bench] {cfg.name}: inputs generated on the GPU in {time.time() - t0:.1f}s")
        kvd = pkv.PKV_BF16 if cfg.dtype == "bf16" else pkv.PKV_F32
        self.pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, kvd)
        tab = self.w.table()
        for g in range(cfg.hkv):
            pkv.pkv_page_table_set(self.pool, 0, g, tab[g])
        self.sparse = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local) if cfg.sparse else None
        dt = self.w.dtype
        self.bufs = {}
        for ch in self.chunks:
            n = ch["q"].shape[0]
            if n not in self.bufs:
                self.bufs[n] = ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page, dt, self.sparse)
        self.sel_counts = {}

    def step(self, keep_counts: bool = False, on_chunk=None):
        """One layer step; on_chunk(c, buffers) is called after chunk c's
        backward is enqueued (the buffers are reused by the next chunk)."""
        pkv, cfg = self.pkv, self.cfg
        pkv.pkv_pool_reset(self.pool, 0)
        pkv.pkv_grad_zero(self.pool, 0)
        for ch in self.chunks:
            pkv.pkv_append_kv(self.pool, 0, ch["q_pos0"], ch["k"], ch["v"])
        for c in reversed(range(len(self.chunks))):
            ch = self.chunks[c]
            b = self.bufs[ch["q"].shape[0]]
            if self.sparse is not None:
                pkv.pkv_select_topk_pages(self.pool, 0, ch["q_pos0"], ch["q"], self.sparse.top_k,
                                          b.sel[0], b.sel[1], self.sparse.n_sink,
                                          self.sparse.n_local)
                if keep_counts:
                    self.sel_counts[c] = b.sel[1].cpu().numpy()
            pkv.pkv_attn_fwd(self.pool, 0, ch["q_pos0"], ch["q"], b.o, b.lse, cfg.scale, sel=b.sel)
            pkv.pkv_attn_bwd(self.pool, 0, ch["q_pos0"], ch["q"], b.o, ch["do"], b.lse, b.dq,
                             cfg.scale, sel=b.sel)
            if on_chunk is not None:
                on_chunk(c, b)

    def pairs(self) -> int:
        """Attended (query, key) pairs summed over query heads, one step."""
        cfg = self.cfg
        if self.sparse is None:
            N = cfg.n_ctx
            return cfg.hq * N * (N + 1) // 2
        return sum(sparse_pairs(self.sel_counts[c], self.chunks[c]["q"].shape[0], cfg.page,
                                cfg.group) for c in range(len(self.chunks)))

    def run(self, steps: int, warmup: int):
        """Step time of `steps` steps (the library's normal mode: dQ and dK/dV
        side by side), then the per-kernel HIP-event times of `steps` more
        steps with kernel timing on (dQ and dK/dV one after the other, so each
        kernel's events bracket its own work)."""
        import torch
        pkv = self.pkv
        for i in range(warmup):
            self.step(keep_counts=(i == 0))
        if warmup == 0:
            self.step(keep_counts=True)
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        marks[0].record()
        for i in range(steps):
            self.step()
            marks[i + 1].record()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        self.step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
        pkv.pkv_kernel_timing(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ktimes = pkv.pkv_kernel_times()
        pkv.pkv_kernel_timing(False)
        return ms, ktimes


def kernel_table(lb: LayerBench, ms_step: float, ktimes: dict, steps: int) -> dict:
    cfg = lb.cfg
    pairs = lb.pairs()
    out = {}
    for k, (tot, n) in ktimes.items():
        if n == 0:
            continue
        e = {"launches_per_step": n // steps, "avg_ms": tot / n, "ms_per_step": tot / steps}
        if k in KERNEL_FLOPS_PER_PAIR:
            # pairs are already x Hq
            e["tflops_executed"] = KERNEL_FLOPS_PER_PAIR[k] * cfg.d * pairs * steps / (tot * 1e-3) / 1e12
            e["tflops_algorithmic"] = (KERNEL_FLOPS_ALGORITHMIC[k] * cfg.d * pairs * steps
                                       / (tot * 1e-3) / 1e12)
        out[k] = e
    return out


def topk_sweep(name: str, budgets, sample_chunks=(63, 40, 16), steps: int = 2) -> list:
    """Step time and the error of the top-K restriction against dense causal
    attention on the same inputs, for several top-K budgets: O and dQ of the
    sampled chunks and the whole dK/dV pool, max |sparse - dense| / max
    |dense|.  Both sides are library outputs (each pinned to the oracle by
    the parity tests); the selection is held constant in the gradients."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    base = get_config_checked(name)

    def run(cfg):
        lb = LayerBench(cfg)
        ms, _ = lb.run(steps, 1)
        keep = {}

        def grab(c, b):
            if c in sample_chunks:
                keep[c] = (b.o.float().clone(), b.dq.clone())
        lb.step(on_chunk=grab)
        n = cfg.n_ctx
        dk = torch.empty(n, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(lb.pool, 0, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(lb.pool, 0, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        pairs = lb.pairs()
        lb.pool.close()
        del lb
        return ms, pairs, keep, dk, dv

    def rel(a, b):
        return float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))

    d_ms, d_pairs, d_keep, d_dk, d_dv = run(base.replace(name=f"{name}@dense", sparse=False))
    out = [{"top_k": "dense", "ms_per_step": round(d_ms, 3), "pairs_frac": 1.0}]
    for k in budgets:
        ms, pairs, keep, dk, dv = run(base.replace(name=f"{name}@K{k}", top_k=k))
        err = {"O": max(rel(keep[c][0], d_keep[c][0]) for c in keep),
               "dq": max(rel(keep[c][1], d_keep[c][1]) for c in keep),
               "dk": rel(dk, d_dk), "dv": rel(dv, d_dv)}
        out.append({"top_k": k, "ms_per_step": round(ms, 3), "pairs_frac": round(pairs / d_pairs, 4),
                    "rel_err_vs_dense": {e: round(v, 4) for e, v in err.items()}})
        log(f"[bench] top-K sweep {name} K={k}: {out[-1]}")
    return out


def get_config_checked(name: str):
    from synthetic import get_config
    return get_config(name)


def phase_rates(lb: "LayerBench", reps: int = 3) -> dict:
    """Data movement of two phases on the largest chunk of a dense workload,
    without arithmetic (libpkv measurement kernels), beside the attention
    kernels of the same chunk:
      * the forward's K/V tile stream into LDS: pkv_measure_gather vs
        pkv_attn_fwd, bytes = the tiles streamed (64 keys x 256 B, K and V,
        per query block and head);
      * the dK/dV atomic epilogue: pkv_measure_atomics over every key, bytes
        = 4 B per fp32 atomic add (dK and dV)."""
    import torch
    pkv, cfg = lb.pkv, lb.cfg
    c = max(range(len(lb.chunks)), key=lambda i: lb.chunks[i]["q_pos0"] * lb.chunks[i]["q"].shape[0])
    ch = lb.chunks[c]
    q_pos0, n_q = ch["q_pos0"], ch["q"].shape[0]
    b = lb.bufs[n_q]
    nqb = -(-n_q // 128)
    tiles = sum((q_pos0 + min(r0 + 128, n_q) - 1 + 64) // 64 for r0 in range(0, n_q, 128))
    gather_bytes = tiles * cfg.hq * 64 * 256 * 2
    out = torch.empty(nqb * cfg.hq, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_g = timed(lambda: pkv.pkv_measure_gather(lb.pool, 0, q_pos0, n_q, cfg.hq, out))
    t_f = timed(lambda: pkv.pkv_attn_fwd(lb.pool, 0, q_pos0, ch["q"], b.o, b.lse, cfg.scale))
    n_keys = cfg.n_ctx
    a_reps = 8
    t_a = timed(lambda: pkv.pkv_measure_atomics(lb.pool, 0, n_keys, a_reps))
    atom_bytes = n_keys * cfg.hkv * cfg.d * 4 * 2 * a_reps
    pkv.pkv_grad_zero(lb.pool, 0)
    torch.cuda.synchronize()
    out = {"chunk": f"rows {q_pos0}..{q_pos0 + n_q - 1}",
           "gather": {"tile_bytes": gather_bytes, "ms": round(t_g, 3),
                      "l2_to_lds_gb_per_s": round(gather_bytes / t_g / 1e6, 1),
                      "fwd_ms_same_chunk": round(t_f, 3),
                      "fwd_l2_to_lds_gb_per_s": round(gather_bytes / t_f / 1e6, 1)},
           "atomics": {"adds": n_keys * cfg.hkv * cfg.d * 2 * a_reps, "ms": round(t_a, 3),
                       "add_gb_per_s": round(atom_bytes / t_a / 1e6, 1),
                       "add_bytes_frac_of_hbm_peak": round(atom_bytes / t_a / 1e6 / PEAK_HBM_GBS, 4)}}
    # HBM bytes the two measurement kernels moved (rocprofv3 FETCH_SIZE /
    # WRITE_SIZE, profiles/traffic.json), as a rate and a fraction of 8 TB/s
    for phase, kern, t in (("gather", "gather", t_g), ("atomics", "atomics", t_a)):
        tb = traffic_for(kern, cfg.name)
        out[phase]["hbm_bytes"] = tb
        if tb:
            out[phase]["hbm_gb_per_s"] = round(tb / t / 1e6, 1)
            out[phase]["hbm_frac_of_peak"] = round(tb / t / 1e6 / PEAK_HBM_GBS, 4)
    return out


def block_bench(n_ctx: int, chunk: int, top_k: int = 0) -> dict:
    """Chunk-recurrent training of one random-initialised Qwen2.5-7B-shaped
    attention block (hidden 3584, Hq 28, Hkv 4, d 128, RoPE base 1e6; bf16
    products, fp32 master weights): forward sweep (appends), backward sweep
    (recompute + attention backward into the pool + the chunks' K/V
    gradients back through W_k, W_v).  Reports time, the attention kernels'
    share, and memory: pool bytes per token and each sweep's transient working
    set (the torch allocator's peak above what stays allocated after it)."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from paged_kv_cache_chunk_amd.recurrent import AttentionBlock

    torch.cuda.empty_cache()
    sparse = Sparse(top_k) if top_k else None
    block = AttentionBlock(max_tokens=n_ctx, sparse=sparse, seed=0)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    xs, gys = [], []
    for p0 in range(0, n_ctx, chunk):
        n = min(chunk, n_ctx - p0)
        xs.append(torch.randn(n, block.hidden, generator=g, device="cuda").to(torch.bfloat16))
        gys.append((torch.randn(n, block.hidden, generator=g, device="cuda") / 64).to(torch.bfloat16))
    block.forward_sweep(xs)      # warm-up
    block.backward_sweep(xs, gys)
    for w in block.parameters():
        w.grad = None
    torch.cuda.synchronize()
    pkv.pkv_kernel_timing(True)
    # transient working set of a sweep = its peak above what stays allocated
    # after it (inputs, outputs kept for the caller, weights and their grads)
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    ys = block.forward_sweep(xs)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ws_fwd = torch.cuda.max_memory_allocated() - torch.cuda.memory_allocated()
    del ys
    torch.cuda.reset_peak_memory_stats()
    dxs = block.backward_sweep(xs, gys)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    ws_bwd = torch.cuda.max_memory_allocated() - torch.cuda.memory_allocated()
    del dxs
    kt = pkv.pkv_kernel_times()
    pkv.pkv_kernel_timing(False)
    attn_ms = sum(kt[k][0] for k in ("select", "fwd", "delta", "dq", "dkdv"))
    pool_b = block.pool_bytes()
    block.close()
    return {"context": n_ctx, "chunk": chunk, "top_k": top_k or None,
            "forward_sweep_s": round(t1 - t0, 3), "backward_sweep_s": round(t2 - t1, 3),
            "tokens_per_s": round(n_ctx / (t2 - t0), 1),
            "attention_kernels_share": round(attn_ms / 1e3 / (t2 - t0), 3),
            "pool_bytes": pool_b, "pool_bytes_per_token": round(pool_b / n_ctx, 1),
            "forward_sweep_working_set_bytes": ws_fwd, "backward_sweep_working_set_bytes": ws_bwd}


def stack_bench(n_layers: int, n_ctx: int, chunk: int, top_k: int = 0,
                host_grads: str = "f32", host_adds: bool = False) -> dict:
    """Chunk-recurrent training of a stack of n_layers random-initialised
    Qwen2.5-7B-shaped attention blocks (hidden 3584, Hq 28, Hkv 4, d 128),
    once with every pool in HBM and once with every layer's K/V (bf16) and
    KV gradients (host_grads: fp32 or bf16) in pinned host memory and two HBM
    windows filled one layer ahead on a side stream (host_adds: gradient
    contributions added into the host tier by the library's host threads, so
    the backward fetches K/V only).  Reports each sweep's time, the overhead of
    the host tier, the copy kernels' time and the share of it hidden behind
    compute (copy time minus the added wall time, over copy time), and the
    HBM and pinned bytes of the pools."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from paged_kv_cache_chunk_amd.recurrent import AttentionStack

    out = {"layers": n_layers, "context": n_ctx, "chunk": chunk, "top_k": top_k or None,
           "host_grad_dtype": host_grads, "host_grad_accumulate": int(host_adds)}
    for mode in ("resident", "host_tier"):
        torch.cuda.empty_cache()
        st = AttentionStack(n_layers, max_tokens=n_ctx, sparse=Sparse(top_k) if top_k else None,
                            seed=0, host_tier=mode == "host_tier",
                            host_grad_dtype=pkv.PKV_BF16 if host_grads == "bf16" else pkv.PKV_F32,
                            host_grad_accumulate=host_adds)
        g = torch.Generator(device="cuda")
        g.manual_seed(11)
        xs, gys = [], []
        for p0 in range(0, n_ctx, chunk):
            n = min(chunk, n_ctx - p0)
            xs.append(torch.randn(n, 3584, generator=g, device="cuda").to(torch.bfloat16))
            gys.append((torch.randn(n, 3584, generator=g, device="cuda") / 64).to(torch.bfloat16))
        st.forward_sweep(xs)  # warm-up step
        st.backward_sweep(xs, gys)
        for w in st.parameters():
            w.grad = None
        torch.cuda.synchronize()
        pkv.pkv_kernel_timing(True)
        torch.cuda.reset_peak_memory_stats()
        t0 = time.perf_counter()
        st.forward_sweep(xs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st.backward_sweep(xs, gys)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        kt = pkv.pkv_kernel_times()
        pkv.pkv_kernel_timing(False)
        dev_b, host_b = st.pool_bytes()
        peak = torch.cuda.max_memory_allocated()
        out[mode] = {"forward_sweep_s": round(t1 - t0, 3), "backward_sweep_s": round(t2 - t1, 3),
                     "tokens_per_s": round(n_ctx / (t2 - t0), 1),
                     "fetch_ms": round(kt["fetch"][0], 1), "writeback_ms": round(kt["writeback"][0], 1),
                     "attention_kernels_ms": round(sum(kt[k][0] for k in ("select", "fwd", "delta",
                                                                           "dq", "dkdv")), 1),
                     "pool_hbm_bytes": dev_b, "pool_host_bytes": host_b,
                     "torch_peak_hbm_bytes": peak}
        log(f"[bench] stack {mode}: {out[mode]}")
        st.close()
        del st, xs, gys
    r, o = out["resident"], out["host_tier"]
    wall_r = r["forward_sweep_s"] + r["backward_sweep_s"]
    wall_o = o["forward_sweep_s"] + o["backward_sweep_s"]
    copy_s = (o["fetch_ms"] + o["writeback_ms"]) / 1e3
    out["host_tier_overhead"] = round(wall_o / wall_r - 1, 4)
    out["copy_hidden_share"] = round(max(0.0, (copy_s - (wall_o - wall_r)) / max(copy_s, 1e-9)), 4)
    return out


def gemm_peak_tflops(n: int = 8192, reps: int = 20) -> float:
    """bf16 GEMM rate of the box's BLAS (torch.matmul of two contiguous
    n x n bf16 matrices, fp32 accumulate): a measured ceiling for dense bf16
    MFMA work at the clock the chip holds under that load, reported beside the
    2.5 PFLOP/s data-sheet figure."""
    import torch
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def cpu_baseline(lb: LayerBench, rows: int) -> dict:
    """The fp64 oracle on a bounded sample of the workload: the last `rows`
    query rows of the context (all heads), forward + backward against every
    key, timed on this host; scaled to tokens/s of the whole workload by the
    share of attended pairs the sample covers."""
    import numpy as np
    import torch
    import oracle

    cfg = lb.cfg
    N = cfg.n_ctx
    ks, vs = [], []
    for ch in lb.chunks:
        ks.append(ch["k"].float().cpu().numpy())
        vs.append(ch["v"].float().cpu().numpy())
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    last = lb.chunks[-1]
    q = last["q"][-rows:].float().cpu().numpy()
    do = last["do"][-rows:].float().cpu().numpy()
    q_pos0 = N - rows
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.attn_bwd(q, k, v, do, q_pos0, cfg.scale, cfg.page)
    dt = time.perf_counter() - t0
    sample_pairs = rows * q_pos0 + rows * (rows + 1) // 2
    total_pairs = N * (N + 1) // 2
    return {"value": N * (sample_pairs / total_pairs) / dt, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle fwd+bwd of the last {rows} query rows x {cfg.hq} heads "
                      f"against all {N} keys ({sample_pairs} pairs/head of {total_pairs}); "
                      f"{dt:.1f}s, scaled by the pair share"}


def cpu_baseline_topk(lb: LayerBench, rows: int) -> dict:
    """The fp64 oracle on a bounded sample of the top-K workload: the
    selection of the last chunk's query pages, then forward + backward of the
    last `rows` query rows (all heads) restricted to it, timed on this host;
    scaled to tokens/s of the whole workload by the share of attended pairs
    the sample covers."""
    import numpy as np
    import oracle

    cfg = lb.cfg
    N = cfg.n_ctx
    k = np.concatenate([ch["k"].float().cpu().numpy() for ch in lb.chunks])
    v = np.concatenate([ch["v"].float().cpu().numpy() for ch in lb.chunks])
    last = lb.chunks[-1]
    q_all = last["q"].float().cpu().numpy()
    q_pos0 = last["q_pos0"]
    do = last["do"][-rows:].float().cpu().numpy()
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    sel = oracle.select_pages(q_all, k, q_pos0, cfg.page, cfg.hkv, cfg.top_k, cfg.n_sink,
                              cfg.n_local, score_dtype=np.float32)
    r0 = q_all.shape[0] - rows
    sub = sel[r0 // cfg.page:]
    oracle.attn_bwd(q_all[r0:], k, v, do, q_pos0 + r0, cfg.scale, cfg.page, sub)
    dt = time.perf_counter() - t0
    counts = np.array([[len(x) for x in row] for row in sub])
    sample_pairs = sparse_pairs(counts, rows, cfg.page, cfg.group)
    total_pairs = lb.pairs()
    return {"value": N * (sample_pairs / total_pairs) / dt, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle: top-K selection of the last chunk's query pages, then "
                      f"fwd+bwd of the last {rows} query rows x {cfg.hq} heads on it "
                      f"({sample_pairs} attended pairs x heads of {total_pairs}); {dt:.1f}s, "
                      "scaled by the pair share"}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    e = data.get(f"{workload}:{kernel}")
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_launch")


def offload_bench(cfg, steps: int, resident_ab: bool, host_accumulate: int = 0,
                  select_ahead: bool = False, window_slots: int = 0) -> dict:
    """Host-offloaded stack: every layer's K/V and KV-gradient pools in pinned
    host memory (bf16), an HBM window of two layers, the next layer's
    selected pages prefetched on a side stream during the current layer, and
    gradient pages written back asynchronously.  Times the backward sweep
    (chunks last to first, layers last to first: select + prefetch + forward
    + backward + writeback); the forward sweep that appends every chunk's
    K/V to the host tier is untimed setup.  host_accumulate: the window's
    gradients start at zero and the library's host threads add each visit's
    contributions into the host tier (no gradient bytes host -> HBM).
    select_ahead: the selections are made before the timed backward sweep
    (as the forward sweep makes them) and reused by it; their time is
    reported apart.  window_slots: page slots per KV head of each HBM window
    (0: a whole layer)."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, OffloadSweep, Sparse
    from synthetic.gpu import GpuWorkload

    L = cfg.n_layers
    ws = [GpuWorkload(cfg, layer=l) for l in range(L)]
    sp = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local) if cfg.sparse else None
    results = {}
    modes = [("offload", 1)] + ([("resident", 0)] if resident_ab else [])
    for mode, host_tier in modes:
        t0 = time.time()
        pool = pkv.pkv_pool_create(L, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                                   pkv.PKV_BF16, host_tier=host_tier, host_grad_dtype=pkv.PKV_BF16,
                                   device_budget_bytes=cfg.hbm_cap_bytes if host_tier else 0,
                                   host_grad_accumulate=host_accumulate if host_tier else 0,
                                   window_slots=window_slots if host_tier else 0)
        dev_b, host_b = pkv.pkv_pool_bytes(pool)
        for l in range(L):
            tab = ws[l].table()
            for g in range(cfg.hkv):
                pkv.pkv_page_table_set(pool, l, g, tab[g])
        log(f"[bench] {cfg.name} {mode}: pool created in {time.time() - t0:.1f}s "
            f"(HBM {dev_b / 2**30:.2f} GiB, pinned host {host_b / 2**30:.2f} GiB)")
        t0 = time.time()
        for c in range(cfg.n_chunks):
            for l in range(L):
                kv = ws[l].chunk(c, "kv")
                pkv.pkv_append_kv(pool, l, kv["q_pos0"], kv["k"], kv["v"])
            if c % 16 == 15:
                torch.cuda.synchronize()
                log(f"[bench] {cfg.name} {mode}: appended chunk {c + 1}/{cfg.n_chunks}")
        torch.cuda.synchronize()
        log(f"[bench] {cfg.name} {mode}: forward-sweep appends in {time.time() - t0:.1f}s")
        sweep = OffloadSweep(pool, L, cfg.hq, cfg.hkv, cfg.d, cfg.page, cfg.scale, sp,
                             torch.bfloat16)
        bufsets = {}

        def inputs(l, c):
            return ws[l].chunk(c, "qd")

        chunk_ids = list(reversed(range(cfg.n_chunks)))[:steps] if steps > 0 else \
            list(reversed(range(cfg.n_chunks)))
        select_s = None
        if sp is not None and select_ahead:
            # the forward sweep's selections, reused by the backward sweep
            torch.cuda.synchronize()
            t_sel = time.perf_counter()
            sweep.select_all(range(L), chunk_ids, inputs)
            torch.cuda.synchronize()
            select_s = time.perf_counter() - t_sel
            log(f"[bench] {cfg.name} {mode}: selections of {len(chunk_ids)} chunks x {L} layers "
                f"made ahead in {select_s:.2f}s")
        pkv.pkv_kernel_timing(True)
        torch.cuda.synchronize()
        windows = []  # (first chunk id of the window, chunks done, bytes fetched, written) so far
        t0 = time.perf_counter()
        def bufs_for(c):
            n = cfg.chunk_range(c)[1]
            if n not in bufsets:
                bufsets[n] = {l: ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page,
                                              torch.bfloat16, sp) for l in range(2)}
            return {l: bufsets[n][l % 2] for l in range(L)}

        for n_done, c in enumerate(chunk_ids):
            # the next chunk's top layer is selected and prefetched during this
            # chunk's layer 0
            nxt = chunk_ids[n_done + 1] if n_done + 1 < len(chunk_ids) else None
            sweep.chunk(c, inputs, bufs_for(c),
                        next_chunk=(nxt, bufs_for(nxt)) if nxt is not None else None)
            if n_done % 8 == 7:
                torch.cuda.synchronize()
                fb, wb = pkv.pkv_offload_bytes(pool)
                windows.append((c, n_done + 1, fb, wb))
                log(f"[bench] {cfg.name} {mode}: backward sweep chunk {n_done + 1}/"
                    f"{len(chunk_ids)}, {time.perf_counter() - t0:.1f}s, "
                    f"fetched {fb / 1e9:.1f} GB, written back {wb / 1e9:.1f} GB")
        torch.cuda.synchronize()
        pkv.pkv_offload_bytes(pool)  # returns after the pending host gradient adds
        wall = time.perf_counter() - t0
        kt = pkv.pkv_kernel_times()
        pkv.pkv_kernel_timing(False)
        fetched, written = pkv.pkv_offload_bytes(pool)
        compute = sum(kt[k][0] for k in ("select", "fwd", "delta", "dq", "dkdv")) / 1e3
        copy = sum(kt[k][0] for k in ("fetch", "writeback")) / 1e3
        per_window = []
        prev = (0, 0, 0)
        for c_last, done, fb, wb in windows:
            n = done - prev[0]
            per_window.append({"chunks": f"{c_last + n - 1}..{c_last}",
                               "fetched_gb_per_layer_chunk": round((fb - prev[1]) / 1e9 / (n * L), 3),
                               "written_gb_per_layer_chunk": round((wb - prev[2]) / 1e9 / (n * L), 3)})
            prev = (done, fb, wb)
        results[mode] = {"wall_s": wall, "compute_kernels_s": compute, "copy_kernels_s": copy,
                         "select_ahead_s": select_s,
                         "per_window": per_window,
                         "fetched_bytes": fetched, "written_bytes": written,
                         "chunks": len(chunk_ids), "hbm_bytes": dev_b, "host_bytes": host_b,
                         "kernels": {k: round(v[0], 1) for k, v in kt.items() if v[1]}}
        log(f"[bench] {cfg.name} {mode}: {results[mode]}")
        pool.close()
        torch.cuda.empty_cache()
    off = results["offload"]
    tokens = sum(cfg.chunk_range(c)[1] for c in (list(reversed(range(cfg.n_chunks)))[:steps]
                                                  if steps > 0 else range(cfg.n_chunks)))
    out = {
        "workload": f"{cfg.name}: {L} layers, {cfg.n_ctx} tokens, chunks of {cfg.chunk}, "
                    + (f"top-K {cfg.top_k} + {cfg.n_sink} sink + {cfg.n_local} local pages"
                       if cfg.sparse else "dense causal")
                    + ", K/V and gradient pools in pinned host memory (bf16), "
                    + (f"two HBM windows of {window_slots} page slots per KV head" if window_slots
                       else "HBM window of 2 layers")
                    + (", gradient contributions added on the host" if host_accumulate else
                       ", gradients accumulated in HBM"),
        "host_grad_accumulate": host_accumulate,
        "selections_made_ahead_s": (round(off["select_ahead_s"], 3)
                                    if off["select_ahead_s"] is not None else None),
        "chunks_timed": off["chunks"],
        "tokens_per_s_per_layer": round(tokens * L / off["wall_s"], 1),
        "backward_sweep_s": round(off["wall_s"], 3),
        "compute_kernels_s": round(off["compute_kernels_s"], 3),
        "copy_kernels_s": round(off["copy_kernels_s"], 3),
        # host link busy time: fetches (host -> HBM) and writebacks (HBM -> host)
        # run on two streams, one per direction of the link
        "link_s": round(max(off["kernels"].get("fetch", 0), off["kernels"].get("writeback", 0)) / 1e3, 3),
        "fetched_gb": round(off["fetched_bytes"] / 1e9, 3),
        "written_back_gb": round(off["written_bytes"] / 1e9, 3),
        "fetch_gbs": round(off["fetched_bytes"] / 1e9 / max(off["kernels"].get("fetch", 0) / 1e3, 1e-9), 1),
        "writeback_gbs": round(off["written_bytes"] / 1e9 / max(off["kernels"].get("writeback", 0) / 1e3, 1e-9), 1),
        "hbm_gib": round(off["hbm_bytes"] / 2**30, 3),
        "host_gib": round(off["host_bytes"] / 2**30, 3),
        "kernels_ms": off["kernels"],
        "bytes_per_8_chunks": off["per_window"],
    }
    if "resident" in results:
        res_s = results["resident"]["wall_s"]
        link = out["link_s"]
        out["resident_s"] = round(res_s, 3)
        out["offload_overhead"] = round(off["wall_s"] / res_s - 1, 4)
        # share of the link time hidden behind compute, and the most that
        # could be hidden (all compute overlapped): min(1, resident / link)
        out["overlap"] = round(max(0.0, (link - (off["wall_s"] - res_s)) / max(link, 1e-9)), 4)
        out["overlap_bound"] = round(min(1.0, res_s / max(link, 1e-9)), 4)
    return out


def roofline_of(ktab: dict, workload: str) -> dict:
    """MFMA roofline of the kernel with the largest time per step: its
    executed FLOP (per attended pair, x pairs) over its summed launch times."""
    dom = max((k for k in ktab if k in KERNEL_FLOPS_PER_PAIR), key=lambda k: ktab[k]["ms_per_step"])
    achieved = ktab[dom]["tflops_executed"]
    return {"bound": "mfma", "kernel": f"{dom}_bf16_kernel", "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(dom, workload),
            "flops_per_pair": f"{KERNEL_FLOPS_PER_PAIR[dom]}*d*Hq"}


def summarize_trace(trace_dir: str) -> dict:
    """Per-kernel totals and copy/compute overlap of a rocprofv3 kernel trace
    (--kernel-trace --output-format csv): for each host-link copy kernel
    (fetch_kernel, writeback_kernel, and the runtime's copy kernel that makes
    the host-adds writeback's contiguous copies and the small list copies),
    the share of its duration during which at least one other kernel runs,
    from the trace's start/end timestamps."""
    import bisect
    import collections
    import csv
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    if not rows:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    copy_names = ("fetch_kernel", "writeback_kernel", "__amd_rocclr_copyBuffer")

    def copy_kind(n):
        return next((c for c in copy_names if c in n), None)

    def merge(iv):
        out = []
        for a, b in sorted(iv):
            if out and a <= out[-1][1]:
                out[-1][1] = max(out[-1][1], b)
            else:
                out.append([a, b])
        return out
    comp = merge((a, b) for n, a, b in rows if copy_kind(n) is None)
    starts = [m[0] for m in comp]

    def covered(a, b):
        tot, i = 0, max(0, bisect.bisect_right(starts, a) - 1)
        while i < len(comp) and comp[i][0] < b:
            x, y = max(a, comp[i][0]), min(b, comp[i][1])
            tot += max(0, y - x)
            i += 1
        return tot
    kern = collections.defaultdict(lambda: [0, 0])
    for n, a, b in rows:
        short = n.replace("void ", "").replace("pkv::(anonymous namespace)::", "")
        short = short[:60] if short.startswith("at::") else short.split("(")[0]
        kern[short][0] += 1
        kern[short][1] += b - a
    out = {"span_s": (max(b for _, _, b in rows) - min(a for _, a, _ in rows)) / 1e9,
           "compute_busy_s": sum(b - a for a, b in comp) / 1e9, "copy": {}, "kernels": {}}
    for c in copy_names:
        iv = [(a, b) for n, a, b in rows if copy_kind(n) == c]
        if not iv:
            continue
        tot = sum(b - a for a, b in iv)
        cov = sum(covered(a, b) for a, b in iv)
        out["copy"][c] = {"launches": len(iv), "summed_s": tot / 1e9,
                          "concurrent_with_compute_s": cov / 1e9, "overlap": cov / max(tot, 1)}
    for k, (n, t) in sorted(kern.items(), key=lambda x: -x[1][1]):
        out["kernels"][k] = {"calls": n, "total_ms": t / 1e6, "avg_ms": t / 1e6 / n}
    return out


def summarize_counters(fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str,
                       workload: str, cal_bytes: int = 1 << 30) -> dict:
    """HBM bytes per launch of the library's kernels from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what
    the same counter reads for a plain device copy of cal_bytes (bench.py
    --copy-calibration); merged into profiles/traffic.json under
    '<workload>:<kernel>' with the current kernel source hash."""
    import collections
    import csv

    def read(d, counter):
        acc = collections.defaultdict(list)
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc
    cf, cw = read(cal_fetch_dir, "FETCH_SIZE"), read(cal_write_dir, "WRITE_SIZE")
    ck = next(k for k in cf if "copyBuffer" in k or "copy" in k.lower())
    ff = cal_bytes / 1024 / (sum(cf[ck]) / len(cf[ck]))
    wf = cal_bytes / 1024 / (sum(cw[ck]) / len(cw[ck]))
    f, w = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    names = {"fwd": "fwd_bf16_kernel", "fwd_merge": "fwd_merge_kernel", "dq": "dq_bf16_kernel",
             "dkdv": "dkdv_bf16_kernel", "gather": "gather_kernel", "atomics": "atomics_kernel"}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data.update({"_doc": "HBM bytes per launch = FETCH_SIZE*fetch_factor + WRITE_SIZE*write_factor "
                         "(KiB -> bytes), averaged over every launch of the profiled run; factors "
                         "from a 1 GiB device copy under the same counters",
                 "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)})
    h = source_hash()
    for key, pat in names.items():
        ks = [k for k in f if pat in k]
        if not ks:
            continue
        fv = [x for k in ks for x in f[k]]
        wv = [x for k in ks for x in w.get(k, [])]
        fk, wk = sum(fv) / len(fv), (sum(wv) / len(wv) if wv else 0.0)
        data[f"{workload}:{key}"] = {"source_hash": h, "bytes_per_launch": int(1024 * (fk * ff + wk * wf)),
                                     "fetch_kib": int(fk), "write_kib": int(wk), "launches": len(fv)}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1)
    return data


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen_128k_dense")
    ap.add_argument("--sparse-workload", default="qwen_256k_topk",
                    help="second workload in the same line ('none' to skip)")
    ap.add_argument("--cpu-rows", type=int, default=384,
                    help="query rows in the oracle's CPU sample (0 skips it)")
    ap.add_argument("--layers", type=int, default=0,
                    help="offloaded workload: number of layers (default: the config's)")
    ap.add_argument("--chunks", type=int, default=0,
                    help="offloaded workload: time only the last N chunks of the backward sweep")
    ap.add_argument("--host-accumulate", type=int, default=0, choices=(0, 1),
                    help="offloaded workload: add gradient contributions on the host instead of "
                         "fetching the gradients into HBM")
    ap.add_argument("--select-ahead", action="store_true",
                    help="offloaded top-K workload: make every selection before the timed backward "
                         "sweep (as the forward sweep does) and reuse them")
    ap.add_argument("--context", type=int, default=0,
                    help="offloaded workload: context length in tokens (default: the config's)")
    ap.add_argument("--window-slots", type=int, default=0,
                    help="offloaded workload: page slots per KV head of each HBM window "
                         "(default: a whole layer)")
    ap.add_argument("--resident-ab", action="store_true",
                    help="offloaded workload: also run the same sweep with all pools in HBM")
    ap.add_argument("--topk-sweep", default="", metavar="K1,K2,..",
                    help="only run the top-K budget sweep on --workload (a top-K workload): "
                         "step time and error against dense attention per budget")
    ap.add_argument("--block", type=int, default=0, metavar="TOKENS",
                    help="only run chunk-recurrent training of one Qwen2.5-7B-shaped attention "
                         "block at TOKENS and TOKENS/2 context (chunks of 12288; --block-top-k K "
                         "for top-K attention)")
    ap.add_argument("--block-top-k", type=int, default=0)
    ap.add_argument("--stack", type=int, default=0, metavar="LAYERS",
                    help="only run chunk-recurrent training of a stack of LAYERS Qwen2.5-7B-shaped "
                         "attention blocks, all pools in HBM vs in the host tier (--stack-ctx, "
                         "--stack-chunk, --block-top-k)")
    ap.add_argument("--stack-ctx", type=int, default=131072)
    ap.add_argument("--stack-chunk", type=int, default=12288)
    ap.add_argument("--stack-host-grads", choices=("f32", "bf16"), default="f32",
                    help="element type of the host tier's KV gradients in --stack")
    ap.add_argument("--stack-host-adds", type=int, default=0,
                    help="1: --stack adds the gradient contributions on the host "
                         "(host_grad_accumulate)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (reference "
                         "for the profiler's FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--summarize-trace", default="", metavar="DIR",
                    help="only print per-kernel totals and copy/compute overlap of a rocprofv3 "
                         "kernel trace under DIR (no GPU)")
    ap.add_argument("--summarize-counters", nargs=5, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "WORKLOAD"),
                    help="only merge rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json "
                         "(no GPU)")
    args = ap.parse_args()

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1), flush=True)
        return
    if args.summarize_counters:
        d = summarize_counters(*args.summarize_counters)
        print(json.dumps({k: v for k, v in d.items() if k.startswith(args.summarize_counters[4])},
                         indent=1), flush=True)
        return

    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from synthetic import get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.stack:
        r = stack_bench(args.stack, args.stack_ctx, args.stack_chunk, args.block_top_k,
                        args.stack_host_grads, bool(args.stack_host_adds))
        print(json.dumps({"metric": "chunk-recurrent attention-stack training: host tier vs HBM",
                          "n_gpus": 1, "dtype": "bf16", "data": "synthetic", **r}), flush=True)
        return
    if args.block:
        runs = [block_bench(n, 12288, args.block_top_k) for n in (args.block // 2, args.block)]
        for r in runs:
            log(f"[bench] block: {r}")
        print(json.dumps({"metric": "chunk-recurrent attention-block training: tokens/s and memory",
                          "n_gpus": 1, "dtype": "bf16", "data": "synthetic", "runs": runs}),
              flush=True)
        return
    cfg = get_config(args.workload)
    if args.topk_sweep:
        budgets = [int(x) for x in args.topk_sweep.split(",")]
        res = topk_sweep(args.workload, budgets)
        print(json.dumps({"metric": "top-K budget sweep: step ms and error vs dense",
                          "workload": args.workload, "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "results": res}), flush=True)
        return
    if cfg.host_tier:
        if args.layers:
            cfg = cfg.replace(n_layers=args.layers)
        if args.context:
            cfg = cfg.replace(n_ctx=args.context, slots=-(-args.context // cfg.page))
        res = offload_bench(cfg, args.chunks, args.resident_ab, args.host_accumulate,
                            args.select_ahead, args.window_slots)
        res.update({"metric": f"offloaded {'top-K' if cfg.sparse else 'dense'} stack: "
                              "backward-sweep tokens/s per layer",
                    "unit": "tokens/s", "n_gpus": 1, "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(res), flush=True)
        return
    lb = LayerBench(cfg)
    log(f"[bench] {cfg.name}: warmup {args.warmup}, timing {args.steps} steps")
    ms, kt = lb.run(args.steps, args.warmup)
    pairs = lb.pairs()
    flops = 14 * cfg.d * pairs
    ktab = kernel_table(lb, ms, kt, args.steps)
    log(f"[bench] {cfg.name}: {ms:.1f} ms/step, {flops / ms / 1e9:.1f} TFLOP/s; kernels {ktab}")

    roofline = roofline_of(ktab, cfg.name)

    line = {
        "metric": "attn fwd+bwd tokens/s per layer, 128K dense & 256K top-K; % bf16 MFMA peak",
        "value": round(cfg.n_ctx / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(sorted(lb.step_ms)[len(lb.step_ms) // 2], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: 1 attention layer, Hq {cfg.hq}, Hkv {cfg.hkv}, "
                               f"d {cfg.d}, {cfg.n_ctx} tokens, chunks of {cfg.chunk}, "
                               f"pages of {cfg.page}, dense causal",
                   "context": cfg.n_ctx, "chunk": cfg.chunk, "page": cfg.page},
        "tflops": round(flops / ms / 1e9, 1),
        "mfma_frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in e.items()}
                    for k, e in ktab.items()},
        "kernel_timing": "HIP events on the launching stream over a second pass of the same steps "
                         "(dQ and dK/dV then run one after the other)",
        "flop_accounting": "tflops and mfma_frac: 14*d*Hq per attended pair (algorithmic); per "
                           "kernel: tflops_executed (fwd 4, dq 6, dkdv 8 x d*Hq: the dQ kernel "
                           "recomputes S and dP) and tflops_algorithmic (fwd 4, dq 2, dkdv 8)",
        "roofline": roofline,
    }

    if not cfg.sparse:
        line["phases"] = phase_rates(lb)
        log(f"[bench] phases: {line['phases']}")
    gemm = gemm_peak_tflops()
    line["gemm_bf16_tflops"] = round(gemm, 1)
    line["mfma_frac_of_gemm"] = round(flops / ms / 1e9 / gemm, 4)
    log(f"[bench] bf16 GEMM (8192^3, torch.matmul): {gemm:.1f} TFLOP/s")

    if args.sparse_workload and args.sparse_workload != "none":
        scfg = get_config(args.sparse_workload)
        del lb
        torch.cuda.empty_cache()
        sb = LayerBench(scfg)
        log(f"[bench] {scfg.name}: warmup {args.warmup}, timing {args.steps} steps")
        sms, skt = sb.run(args.steps, args.warmup)
        spairs = sb.pairs()
        sfl = 14 * scfg.d * spairs
        sktab = kernel_table(sb, sms, skt, args.steps)
        log(f"[bench] {scfg.name}: {sms:.1f} ms/step, {sfl / sms / 1e9:.1f} TFLOP/s; {sktab}")
        line["topk_256k"] = {
            "workload": f"{scfg.name}: {scfg.n_ctx} tokens, chunks of {scfg.chunk}, top-K "
                        f"{scfg.top_k} + {scfg.n_sink} sink + {scfg.n_local} local pages",
            "tokens_per_s": round(scfg.n_ctx / (sms * 1e-3), 1),
            "ms_per_step": round(sms, 3),
            "tflops": round(sfl / sms / 1e9, 1),
            "mfma_frac": round(sfl / sms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "attended_pairs_x_heads": spairs,
            "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                            for kk, vv in e.items()} for k, e in sktab.items()},
            "roofline": roofline_of(sktab, scfg.name),
        }
        if args.cpu_rows:
            rows = max(scfg.page, (args.cpu_rows // 3) // scfg.page * scfg.page)
            log(f"[bench] cpu baseline: oracle on {rows} rows of {scfg.name}")
            line["topk_256k"]["cpu_baseline"] = cpu_baseline_topk(sb, rows)
        del sb
        torch.cuda.empty_cache()
        lb = LayerBench(cfg) if args.cpu_rows else None

    if args.cpu_rows:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows")
        line["cpu_baseline"] = cpu_baseline(lb, args.cpu_rows)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
