"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (whole context, one layer, chunks run in reverse order after every
append), on outputs the oracle can compute one by one:
  * O, LSE, dQ of sampled rows (every chunk's first, middle and last row,
    three query heads);
  * dK, dV of the last keys of the context in full (only the last rows see
    them, so the oracle's cost stays small);
  * at 256K top-K, the last chunk's own dK/dV contribution (the sweep's first
    backward) to the sink page and the three pages its query pages share
    most, every element;
  * for every key, the sums that hold at any size: sum_s dK = 0 and
    sum_s dV = sum of dO over the group's heads and all rows;
  * in top-K mode, the selections (exact, up to the 1e-5 score-gap rule;
    every chunk at 256K) and the sampled rows use the oracle's own selection.
Inputs come from the GPU generator (synthetic.gpu) and are copied back for
the oracle."""
import numpy as np
import pytest

import oracle
from synthetic import get_config
from tests.gpu_util import compare_selection, gpu_available, rel_err, sel_lists

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _run(cfg, sample_rows, sample_heads, sel_chunks=(), shared_pages=0):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, Sparse
    from synthetic.gpu import GpuWorkload

    w = GpuWorkload(cfg)
    chunks = [w.chunk(c) for c in range(cfg.n_chunks)]
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16)
    tab = w.table()
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    sparse = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local) if cfg.sparse else None
    for ch in chunks:
        pkv.pkv_append_kv(pool, 0, ch["q_pos0"], ch["k"], ch["v"])
    samples, sels = {}, {}
    first_pages = None
    for c in reversed(range(len(chunks))):
        ch = chunks[c]
        n = ch["q"].shape[0]
        b = ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page, w.dtype, sparse)
        if sparse is not None:
            pkv.pkv_select_topk_pages(pool, 0, ch["q_pos0"], ch["q"], sparse.top_k, b.sel[0],
                                      b.sel[1], sparse.n_sink, sparse.n_local)
        pkv.pkv_attn_fwd(pool, 0, ch["q_pos0"], ch["q"], b.o, b.lse, cfg.scale, sel=b.sel)
        pkv.pkv_attn_bwd(pool, 0, ch["q_pos0"], ch["q"], b.o, ch["do"], b.lse, b.dq, cfg.scale,
                         sel=b.sel)
        torch.cuda.synchronize()
        rows = sorted({0, n // 2, n - 1} | set(sample_rows(n)))
        ri = torch.tensor(rows, device="cuda")
        samples[c] = dict(rows=rows, O=b.o[ri].float().cpu().numpy(),
                          lse=b.lse[:, ri].cpu().numpy(), dq=b.dq[ri].cpu().numpy())
        if sparse is not None and c in sel_chunks:
            sels[c] = (b.sel[0].cpu().numpy(), b.sel[1].cpu().numpy())
        if shared_pages and c == len(chunks) - 1:
            # the first backward of the sweep: the pool's dK/dV hold this
            # chunk's contribution only.  Keep the sink page and the pages
            # the chunk's query pages share most (many work items, one atomic
            # epilogue each).
            pg, cnt = b.sel[0].cpu().numpy(), b.sel[1].cpu().numpy()
            hits = np.zeros(cfg.n_pages, dtype=np.int64)
            for il in range(pg.shape[0]):
                for g in range(cfg.hkv):
                    hits[pg[il, g, :cnt[il, g]]] += 1
            hits[0] = -1
            shared = [0] + [int(x) for x in np.argsort(-hits, kind="stable")[:shared_pages - 1]]
            first = dict(pages=shared, lists=[int(cnt.size) if p == 0 else int(hits[p])
                                              for p in shared], dk=[], dv=[])
            for p in shared:
                for what, key in ((pkv.PKV_DK, "dk"), (pkv.PKV_DV, "dv")):
                    dst = torch.empty(cfg.page, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
                    pkv.pkv_read_rows(pool, 0, what, p * cfg.page, dst)
                    torch.cuda.synchronize()
                    first[key].append(dst.cpu().numpy())
            first_pages = first
    N = cfg.n_ctx
    dk = torch.empty(N, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dv)
    torch.cuda.synchronize()
    host = dict(k=np.concatenate([ch["k"].float().cpu().numpy() for ch in chunks]),
                v=np.concatenate([ch["v"].float().cpu().numpy() for ch in chunks]))
    do_sum = [sum(ch["do"].double()[:, g * cfg.group:(g + 1) * cfg.group].sum(dim=(0, 1))
                  for ch in chunks).cpu().numpy() for g in range(cfg.hkv)]
    pool.close()
    return dict(chunks=chunks, samples=samples, sels=sels, dk=dk.cpu().numpy(),
                dv=dv.cpu().numpy(), do_sum=do_sum, first_pages=first_pages, **host)


def _oracle_sel(cfg, got, c):
    ch = got["chunks"][c]
    q = ch["q"].float().cpu().numpy()
    return oracle.select_pages(q, got["k"], ch["q_pos0"], cfg.page, cfg.hkv, cfg.top_k,
                               cfg.n_sink, cfg.n_local, score_dtype=np.float32,
                               return_scores=True)


def _check(cfg, got, heads, key_tail, sel_chunks=()):
    k, v = got["k"], got["v"]
    worst = {"O": 0.0, "lse": 0.0, "dq": 0.0}
    osel = {}
    n_diff = 0
    for c in sel_chunks:
        ref_sel, scores = _oracle_sel(cfg, got, c)
        gpu_sel = sel_lists(got["sels"][c])
        # differences only inside the 1e-5 score gap (asserted inside)
        n_diff += compare_selection(gpu_sel, ref_sel, scores, cfg.top_k)
        # values are checked on the GPU's selection, which the rule admits
        osel[c] = [[np.array(lst, dtype=np.int64) for lst in row] for row in gpu_sel]
    if sel_chunks:
        print(f"{cfg.name}: selections of {len(sel_chunks)} chunks checked, {n_diff} lists "
              "differ inside the score gap", flush=True)
    for c, s in got["samples"].items():
        ch = got["chunks"][c]
        if cfg.sparse and c not in osel:
            continue
        rows = np.array(s["rows"])
        t_abs = ch["q_pos0"] + rows
        q = ch["q"].float().cpu().numpy()[rows]
        do = ch["do"].float().cpu().numpy()[rows]
        for h in heads:
            ok = None
            if cfg.sparse:
                ok = np.zeros((len(rows), cfg.n_pages), dtype=bool)
                for n_, r in enumerate(rows):
                    ok[n_, osel[c][r // cfg.page][h // cfg.group]] = True
            O, lse, dq = oracle.rows_fwd_bwd(q[:, h], do[:, h], t_abs, h, k, v, cfg.scale,
                                             cfg.group, cfg.page, ok)
            worst["O"] = max(worst["O"], rel_err(s["O"][:, h], O))
            worst["lse"] = max(worst["lse"], rel_err(s["lse"][h], lse))
            worst["dq"] = max(worst["dq"], rel_err(s["dq"][:, h], dq))
    N = cfg.n_ctx
    s0 = N - key_tail
    last = got["chunks"][-1]
    off = s0 - last["q_pos0"]
    sels = None
    if cfg.sparse:
        sels = {cfg.n_chunks - 1: osel[cfg.n_chunks - 1]}
    dk, dv = oracle.key_grads_sampled(s0, last["q"].float().cpu().numpy()[off:],
                                      last["do"].float().cpu().numpy()[off:], k, v, cfg.scale,
                                      cfg.chunk, cfg.page, sels)
    worst["dk_tail"] = rel_err(got["dk"][s0:], dk)
    worst["dv_tail"] = rel_err(got["dv"][s0:], dv)
    first = got.get("first_pages")
    if first is not None:
        # the last chunk's own contribution to the sink and the most shared
        # pages, every element, against the oracle on the same selection
        pages = first["pages"]
        rdk, rdv = oracle.chunk_page_grads(last["q"].float().cpu().numpy(),
                                           last["do"].float().cpu().numpy(), last["q_pos0"], k, v,
                                           cfg.scale, cfg.page, osel[cfg.n_chunks - 1], pages)
        worst["dk_shared_pages"] = rel_err(np.stack(first["dk"]), rdk)
        worst["dv_shared_pages"] = rel_err(np.stack(first["dv"]), rdv)
        print(f"{cfg.name}: last chunk's dK/dV of pages {pages} (held by {first['lists']} of the "
              f"chunk's (query page, KV head) lists) checked element-wise", flush=True)
    # sums over every key
    for g in range(cfg.hkv):
        sk = np.abs(got["dk"][:, g].astype(np.float64).sum(0)).max()
        scale_k = np.abs(got["dk"][:, g]).astype(np.float64).sum(0).max()
        worst[f"sum_dk_{g}"] = sk / scale_k
        worst[f"sum_dv_{g}"] = rel_err(got["dv"][:, g].astype(np.float64).sum(0), got["do_sum"][g])
    print(cfg.name, {k_: f"{v_:.2e}" for k_, v_ in worst.items()}, flush=True)
    for name, e in worst.items():
        assert e <= 1e-2, f"{name}: {e:.3e}"


def test_qwen_32k_dense_full():
    cfg = get_config("qwen_32k_dense")
    got = _run(cfg, lambda n: [1, 127, 128, 4095 % n], None)
    _check(cfg, got, heads=(0, 13, 27), key_tail=64)


def test_qwen_128k_dense_full():
    cfg = get_config("qwen_128k_dense")
    got = _run(cfg, lambda n: [129], None)
    _check(cfg, got, heads=(0, 27), key_tail=32)


def test_qwen_256k_topk_full():
    """Selections of all 64 chunks (8192 lists) against the oracle's fp32
    scoring; sampled rows of every chunk on the oracle's selection."""
    cfg = get_config("qwen_256k_topk")
    every = tuple(range(cfg.n_chunks))
    got = _run(cfg, lambda n: [128, 2049], None, sel_chunks=every, shared_pages=4)
    _check(cfg, got, heads=(0, 15), key_tail=32, sel_chunks=every)


@pytest.mark.parametrize("accumulate", [0, 1])
def test_qwen_1m_offload_last_chunk(accumulate):
    """The 1M-token top-K workload with every pool in the host tier (2 of its
    28 layers: the per-layer path is the same for every layer, and the box
    pins at most 64 GiB per process): the backward sweep of the last chunk
    through OffloadSweep (select one layer ahead, prefetch on a side stream,
    gradient writeback), checked per layer against the oracle on the
    selection of the chunk, sampled rows (O, LSE, dQ) and the last keys'
    dK/dV in full, which only the last chunk's rows reach.  accumulate=1: the
    gradient contributions are added into the host tier by host threads."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, OffloadSweep, Sparse
    from synthetic.gpu import GpuWorkload

    cfg = get_config("qwen_1m_offload").replace(n_layers=2)
    L, c_last = cfg.n_layers, cfg.n_chunks - 1
    ws = [GpuWorkload(cfg, layer=l) for l in range(L)]
    pool = pkv.pkv_pool_create(L, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                               host_tier=1, host_grad_dtype=pkv.PKV_BF16,
                               device_budget_bytes=cfg.hbm_cap_bytes,
                               host_grad_accumulate=accumulate)
    for l in range(L):
        tab = ws[l].table()
        for g in range(cfg.hkv):
            pkv.pkv_page_table_set(pool, l, g, tab[g])
    host_k = [[] for _ in range(L)]
    host_v = [[] for _ in range(L)]
    for c in range(cfg.n_chunks):
        for l in range(L):
            kv = ws[l].chunk(c, "kv")
            pkv.pkv_append_kv(pool, l, kv["q_pos0"], kv["k"], kv["v"])
            host_k[l].append(kv["k"].float().cpu().numpy())
            host_v[l].append(kv["v"].float().cpu().numpy())
    sp = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local)
    sweep = OffloadSweep(pool, L, cfg.hq, cfg.hkv, cfg.d, cfg.page, cfg.scale, sp, torch.bfloat16)
    ins = {l: ws[l].chunk(c_last, "qd") for l in range(L)}
    n = ins[0]["q"].shape[0]
    bufs = {l: ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page, torch.bfloat16, sp)
            for l in range(L)}
    rows = sorted({0, 1, 127, 128, n // 2, n - 1})
    got = {}

    def outputs(l, c, b):
        ri = torch.tensor(rows, device="cuda")
        got[l] = dict(O=b.o[ri].float().cpu().numpy(), lse=b.lse[:, ri].cpu().numpy(),
                      dq=b.dq[ri].cpu().numpy(),
                      sel=(b.sel[0].cpu().numpy(), b.sel[1].cpu().numpy()))

    sweep.chunk(c_last, lambda l, c: ins[l], bufs, outputs)
    torch.cuda.synchronize()
    N, tail = cfg.n_ctx, 32
    worst = {}
    for l in range(L):
        dk = torch.empty(N, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(pool, l, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, l, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        k = np.concatenate(host_k[l])
        v = np.concatenate(host_v[l])
        q = ins[l]["q"].float().cpu().numpy()
        do = ins[l]["do"].float().cpu().numpy()
        q_pos0 = ins[l]["q_pos0"]
        ref_sel, scores = oracle.select_pages(q, k, q_pos0, cfg.page, cfg.hkv, cfg.top_k,
                                              cfg.n_sink, cfg.n_local, score_dtype=np.float32,
                                              return_scores=True)
        gpu_sel = sel_lists(got[l]["sel"])
        nd = compare_selection(gpu_sel, ref_sel, scores, cfg.top_k)
        print(f"layer {l}: {nd} lists differ inside the score gap", flush=True)
        ref_sel = [[np.array(lst, dtype=np.int64) for lst in row] for row in gpu_sel]
        t_abs = q_pos0 + np.array(rows)
        for h in (0, 15, 27):
            ok = np.zeros((len(rows), cfg.n_pages), dtype=bool)
            for i, r in enumerate(rows):
                ok[i, ref_sel[r // cfg.page][h // cfg.group]] = True
            O, lse, dq = oracle.rows_fwd_bwd(q[rows, h], do[rows, h], t_abs, h, k, v, cfg.scale,
                                             cfg.group, cfg.page, ok)
            worst[f"O{l}"] = max(worst.get(f"O{l}", 0.0), rel_err(got[l]["O"][:, h], O))
            worst[f"lse{l}"] = max(worst.get(f"lse{l}", 0.0), rel_err(got[l]["lse"][h], lse))
            worst[f"dq{l}"] = max(worst.get(f"dq{l}", 0.0), rel_err(got[l]["dq"][:, h], dq))
        s0 = N - tail
        off = s0 - q_pos0
        rdk, rdv = oracle.key_grads_sampled(s0, q[off:], do[off:], k, v, cfg.scale, cfg.chunk,
                                            cfg.page, {c_last: ref_sel})
        # bf16 host gradient tier: the tail's grads made one bf16 round trip
        worst[f"dk_tail{l}"] = rel_err(dk.cpu().numpy()[s0:], rdk)
        worst[f"dv_tail{l}"] = rel_err(dv.cpu().numpy()[s0:], rdv)
        del k, v
    pool.close()
    print(cfg.name, f"host adds {accumulate}", {k_: f"{v_:.2e}" for k_, v_ in worst.items()},
          flush=True)
    for name, e in worst.items():
        assert e <= 1e-2, f"{name}: {e:.3e}"


def test_four_million_token_layer_last_chunk():
    """One layer of the top-K workload at a 4,194,304-token context (32768
    pages per KV head) in the host tier, with windows of 64 x 131 = 8384 slots
    per KV head (what a chunk of 8192 tokens with top-K 128 + 3 forced pages
    can name): the pool's HBM stays under the 16 GiB cap, and the backward
    sweep of the last chunk (selection, prefetch of the selected pages and
    their gradients, forward, backward, gradient writeback) matches the
    oracle: the selection of all 64 x 4 lists (1e-5 score-gap rule), O, LSE
    and dQ of sampled rows, and the chunk's dK/dV contributions to the sink
    page and the three pages its query pages share most, every element, after
    their round trip through the bf16 host tier."""
    import time
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, OffloadSweep, Sparse
    from synthetic.gpu import GpuWorkload

    cfg = get_config("qwen_1m_offload").replace(n_ctx=4 << 20, slots=32768, n_layers=1)
    assert cfg.n_pages == 32768 and cfg.n_chunks == 512
    ws = 64 * 131
    w = GpuWorkload(cfg, layer=0)
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                               host_tier=1, host_grad_dtype=pkv.PKV_BF16, window_slots=ws,
                               device_budget_bytes=cfg.hbm_cap_bytes)
    dev_bytes, host_bytes = pkv.pkv_pool_bytes(pool)
    print(f"4M-token layer: pool HBM {dev_bytes / 2**30:.2f} GiB, pinned {host_bytes / 2**30:.2f} GiB",
          flush=True)
    assert dev_bytes < cfg.hbm_cap_bytes
    tab = w.table()
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    k = np.empty((cfg.n_ctx, cfg.hkv, cfg.d), dtype=np.float32)
    v = np.empty_like(k)
    for c in range(cfg.n_chunks):
        kv = w.chunk(c, "kv")
        pkv.pkv_append_kv(pool, 0, kv["q_pos0"], kv["k"], kv["v"])
        lo = kv["q_pos0"]
        k[lo:lo + kv["k"].shape[0]] = kv["k"].float().cpu().numpy()
        v[lo:lo + kv["v"].shape[0]] = kv["v"].float().cpu().numpy()
    c_last = cfg.n_chunks - 1
    ch = w.chunk(c_last, "qd")
    n, q_pos0 = ch["q"].shape[0], ch["q_pos0"]
    sp = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local)
    sweep = OffloadSweep(pool, 1, cfg.hq, cfg.hkv, cfg.d, cfg.page, cfg.scale, sp, torch.bfloat16)
    bufs = {0: ChunkBuffers(n, cfg.hq, cfg.hkv, cfg.d, cfg.page, torch.bfloat16, sp)}
    rows = sorted({0, 1, 127, 128, n // 2, n - 1})
    got = {}

    def outputs(l, c, b):
        ri = torch.tensor(rows, device="cuda")
        got.update(O=b.o[ri].float().cpu().numpy(), lse=b.lse[:, ri].cpu().numpy(),
                   dq=b.dq[ri].cpu().numpy(), sel=(b.sel[0].cpu().numpy(), b.sel[1].cpu().numpy()))

    torch.cuda.synchronize()
    t0 = time.time()
    sweep.chunk(c_last, lambda l, c: ch, bufs, outputs)
    torch.cuda.synchronize()
    print(f"4M-token layer: last chunk's sweep {1e3 * (time.time() - t0):.1f} ms "
          f"(selection, prefetch, forward, backward, writeback; outputs copied to the host)",
          flush=True)
    pg, cnt = got["sel"]
    hits = np.zeros(cfg.n_pages, dtype=np.int64)
    for il in range(pg.shape[0]):
        for g in range(cfg.hkv):
            hits[pg[il, g, :cnt[il, g]]] += 1
    hits[0] = -1
    pages = [0] + [int(x) for x in np.argsort(-hits, kind="stable")[:3]]
    dk_all = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk_all)
    dk = np.stack([dk_all[p * cfg.page:(p + 1) * cfg.page].cpu().numpy() for p in pages])
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dk_all)
    dv = np.stack([dk_all[p * cfg.page:(p + 1) * cfg.page].cpu().numpy() for p in pages])
    del dk_all
    pool.close()
    q = ch["q"].float().cpu().numpy()
    do = ch["do"].float().cpu().numpy()
    ref_sel, scores = oracle.select_pages(q, k, q_pos0, cfg.page, cfg.hkv, cfg.top_k, cfg.n_sink,
                                          cfg.n_local, score_dtype=np.float32, return_scores=True)
    gpu_sel = sel_lists(got["sel"])
    nd = compare_selection(gpu_sel, ref_sel, scores, cfg.top_k)
    sel = [[np.array(lst, dtype=np.int64) for lst in row] for row in gpu_sel]
    worst = {"O": 0.0, "lse": 0.0, "dq": 0.0}
    t_abs = q_pos0 + np.array(rows)
    for h in (0, 15, 27):
        ok = np.zeros((len(rows), cfg.n_pages), dtype=bool)
        for i, r in enumerate(rows):
            ok[i, sel[r // cfg.page][h // cfg.group]] = True
        O, lse, dq = oracle.rows_fwd_bwd(q[rows, h], do[rows, h], t_abs, h, k, v, cfg.scale,
                                         cfg.group, cfg.page, ok)
        worst["O"] = max(worst["O"], rel_err(got["O"][:, h], O))
        worst["lse"] = max(worst["lse"], rel_err(got["lse"][h], lse))
        worst["dq"] = max(worst["dq"], rel_err(got["dq"][:, h], dq))
    rdk, rdv = oracle.chunk_page_grads(q, do, q_pos0, k, v, cfg.scale, cfg.page, sel, pages)
    worst["dk_shared_pages"] = rel_err(dk, rdk)
    worst["dv_shared_pages"] = rel_err(dv, rdv)
    print(f"4M-token layer: {nd} lists differ inside the score gap; pages {pages} held by "
          f"{[int(cnt.size) if p == 0 else int(hits[p]) for p in pages]} lists;",
          {k_: f"{v_:.2e}" for k_, v_ in worst.items()}, flush=True)
    for name, e in worst.items():
        assert e <= 1e-2, f"{name}: {e:.3e}"
