"""GPU parity: libpkv (HIP, gfx950) against the fp64 oracle on seeded inputs,
at sizes the oracle finishes in seconds (several tiles, ragged last chunk).
Error metric: max |x_gpu - x_ref| / max |x_ref| over the whole tensor.
Bounds: 1e-5 for fp32 pools, 1e-2 for bf16 pools (fp32 accumulation)."""
import numpy as np
import pytest

import oracle
from synthetic import Workload, get_config, mini_config
from tests.gpu_util import compare_selection, gpu_available, rel_err, run_layer, sel_lists

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _oracle_for(cfg, w, sparse=None, score_dtype=np.float32):
    f = w.full()
    sp = None
    if sparse is not None:
        sp = dict(top_k=sparse.top_k, n_sink=sparse.n_sink, n_local=sparse.n_local,
                  score_dtype=score_dtype)
    return f, oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page, sparse=sp)


def _check(cfg, got, ref, tol):
    errs = {name: rel_err(got[name], ref[name]) for name in ("O", "lse", "dq", "dk", "dv")}
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= tol, f"{name}: {e:.3e} > {tol}"
    return errs


def _gpu_sels(cfg, got):
    """The GPU's selections in the oracle's format (per chunk, per query page,
    per KV head: ascending page ids)."""
    out = []
    for c in range(cfg.n_chunks):
        pages, count = got["sel"][c]
        out.append([[pages[i, g, :count[i, g]].astype(np.int64) for g in range(cfg.hkv)]
                    for i in range(pages.shape[0])])
    return out


def _check_sel(cfg, f, got, ref, sparse):
    """Selections of every chunk against the oracle's fp32 scoring, equal
    except for candidates within 1e-5 of the K-th score.  Returns the oracle
    result to compare values with: `ref` when the selections are equal, else
    the oracle run on the GPU's own selections (the gap rule makes each of
    them a correct selection; the attention given a selection is exact)."""
    n_diff = 0
    for c in range(cfg.n_chunks):
        q_pos0, n = cfg.chunk_range(c)
        _, scores = oracle.select_pages(f.q[q_pos0:q_pos0 + n], f.k, q_pos0, cfg.page, cfg.hkv,
                                        sparse.top_k, sparse.n_sink, sparse.n_local,
                                        return_scores=True)
        n_diff += compare_selection(sel_lists(got["sel"][c]), ref["sel"][c], scores, sparse.top_k)
    if n_diff == 0:
        return ref
    print(f"{cfg.name}: {n_diff} lists differ inside the 1e-5 score gap; values checked on "
          "the GPU's selections", flush=True)
    return oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page,
                             sels=_gpu_sels(cfg, got))


def test_tiny_f32_dense():
    cfg = get_config("tiny_f32")
    w = Workload(cfg)
    got = run_layer(cfg, w)
    _, ref = _oracle_for(cfg, w)
    _check(cfg, got, ref, TOL["f32"])


def test_tiny_f32_sparse():
    from paged_kv_cache_chunk_amd.chunks import Sparse
    cfg = get_config("tiny_f32")
    sp = Sparse(top_k=4)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["f32"])


def test_f32_qwen_shape():
    cfg = mini_config("qwen_32k_dense", n_ctx=640, chunk=256).replace(dtype="f32")
    w = Workload(cfg)
    got = run_layer(cfg, w)
    _, ref = _oracle_for(cfg, w)
    _check(cfg, got, ref, TOL["f32"])


def test_bf16_qwen_dense_ragged():
    # 13 pages, chunks of 5 pages with a last chunk of 3; 28/4 heads, d 128
    cfg = mini_config("qwen_32k_dense", n_ctx=1664, chunk=640)
    w = Workload(cfg)
    got = run_layer(cfg, w)
    _, ref = _oracle_for(cfg, w)
    _check(cfg, got, ref, TOL["bf16"])


def test_bf16_qwen_sparse():
    from paged_kv_cache_chunk_amd.chunks import Sparse
    cfg = mini_config("qwen_256k_topk", n_ctx=3072, chunk=1024, top_k=4)
    sp = Sparse(top_k=4)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["bf16"])


def test_bf16_page_table_permutation_invariance():
    cfg = mini_config("qwen_32k_dense", n_ctx=1024, chunk=512)
    w = Workload(cfg)
    ident = np.tile(np.arange(cfg.n_pages, dtype=np.int32), (cfg.hkv, 1))
    a = run_layer(cfg, w, table=ident)
    b = run_layer(cfg, w)
    assert not np.array_equal(ident, w.table())
    for name in ("O", "lse", "dq"):
        assert np.array_equal(a[name], b[name]), name
    for name in ("dk", "dv"):
        assert rel_err(a[name], b[name]) < 1e-5, name


def test_bf16_qwen_dense_partial_page_tail():
    # last chunk of 360 rows: neither a page nor a 32-row tile multiple; the
    # last page holds 104 tokens
    cfg = mini_config("qwen_32k_dense", n_ctx=1000, chunk=640)
    w = Workload(cfg)
    got = run_layer(cfg, w)
    _, ref = _oracle_for(cfg, w)
    _check(cfg, got, ref, TOL["bf16"])


def test_bf16_qwen_sparse_partial_page_tail():
    from paged_kv_cache_chunk_amd.chunks import Sparse
    cfg = mini_config("qwen_256k_topk", n_ctx=2000, chunk=1024, top_k=3)
    sp = Sparse(top_k=3)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["bf16"])


def test_f32_partial_page_tail():
    cfg = get_config("tiny_f32").replace(n_ctx=500)
    w = Workload(cfg)
    got = run_layer(cfg, w)
    _, ref = _oracle_for(cfg, w)
    _check(cfg, got, ref, TOL["f32"])


@pytest.mark.parametrize("n_sink,n_local", [(1, 2), (0, 4), (2, 1)])
def test_bf16_local_window_mode(n_sink, n_local):
    """top_k = 0: the selection is the forced pages only (sink pages and a
    window of the n_local most recent pages), i.e. sliding-window attention
    with attention sinks; no scoring is involved, so the lists are exact."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    cfg = mini_config("qwen_256k_topk", n_ctx=3072, chunk=1024, top_k=0, n_sink=n_sink,
                      n_local=n_local)
    sp = Sparse(top_k=0, n_sink=n_sink, n_local=n_local)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    for c in range(cfg.n_chunks):
        q_pos0, n = cfg.chunk_range(c)
        pages, count = got["sel"][c]
        for il in range(pages.shape[0]):
            i = q_pos0 // cfg.page + il
            want = sorted(set(range(min(n_sink, i + 1))) | set(range(max(0, i - n_local + 1), i + 1)))
            for g in range(cfg.hkv):
                assert list(pages[il, g, :count[il, g]]) == want
    _check(cfg, got, ref, TOL["bf16"])


@pytest.mark.parametrize("hq,hkv,page,sparse_k", [
    (8, 2, 256, 0),    # pages of 256 tokens (two 128-key slabs per page), G = 4
    (8, 2, 256, 3),    # the same in top-K mode
    (4, 4, 128, 0),    # multi-head attention (G = 1)
    (16, 1, 128, 2),   # one KV head for 16 query heads, top-K
])
def test_bf16_other_shapes(hq, hkv, page, sparse_k):
    """bf16 kernels at head ratios and page sizes other than the Qwen
    shape's, with a ragged last chunk, against the oracle."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    base = "qwen_256k_topk" if sparse_k else "qwen_32k_dense"
    n_ctx = 10 * page + page // 2 + 32
    cfg = mini_config(base, n_ctx=n_ctx, chunk=4 * page, hq=hq, hkv=hkv, page=page,
                      top_k=sparse_k)
    sp = Sparse(top_k=sparse_k) if sparse_k else None
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    if sp is not None:
        ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["bf16"])


def _split_plan(units: int):
    """The forward's tail split on this device (two workgroups per compute
    unit): (units split in two, first part's fraction of the key tiles)."""
    import torch
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    if units < slots:
        return 0, None
    r = units % slots
    if r == 0 or 10 * r > 9 * slots:
        return 0, None
    return r, (r / slots if 2 * r >= slots else 0.5)


@pytest.mark.parametrize("n_ctx,chunk,top_k,page", [
    (7168, 3584, 6, 128),  # 2 chunks of 28 query blocks x 28 heads: 784 units, the last 272 split (cut 272/512)
    (2600, 2688, 3, 128),  # one chunk of 21 query blocks (ragged last one): 588 units, 76 split in halves
    (2816, 2816, 3, 256),  # pages of 256 (4 key tiles each, a part may start inside a page): 616 units, 104 split
])
def test_bf16_topk_forward_tail_split(n_ctx, chunk, top_k, page):
    """Top-K chunks large enough that the bf16 forward cuts its last pass of
    work units in two parts along their key tiles (every unit attends about
    as many keys, so a partial last pass would leave slots idle): each part
    keeps a partial softmax state and a second kernel combines the two.  O,
    LSE, dQ, dK, dV against the oracle, every element; and a second run
    bit-identical."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    cfg = mini_config("qwen_256k_topk", n_ctx=n_ctx, chunk=chunk, top_k=top_k, page=page)
    plans = [_split_plan(-(-cfg.chunk_range(c)[1] // 128) * cfg.hq) for c in range(cfg.n_chunks)]
    print(f"splits per chunk: {plans}", flush=True)
    if not any(n for n, _ in plans):
        pytest.skip("no chunk of this case has a split last pass on this device")
    sp = Sparse(top_k=top_k)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    again = run_layer(cfg, w, sparse=sp)
    for name in ("O", "lse", "dq"):
        assert np.array_equal(got[name], again[name]), name
    f, ref = _oracle_for(cfg, w, sp)
    ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["bf16"])
    got["pool"].close()
    again["pool"].close()


def test_bf16_sparse_chunk_over_64_query_pages():
    """A top-K chunk of 71 query pages: the sparse dK/dV work items carry the
    first two 32-bit words of their key page's query-page mask and the kernel
    reads the third from the plan (chunks of more than 64 query pages); the
    sink page, held by every query page, is cut into items of 8."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    n_ctx = 70 * 128 + 40
    cfg = mini_config("qwen_256k_topk", n_ctx=n_ctx, chunk=n_ctx, hq=4, hkv=1, top_k=3)
    sp = Sparse(top_k=3)
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL["bf16"])


@pytest.mark.parametrize("ragged", [False, True])
def test_bf16_topk_covering_every_page_equals_dense(ragged):
    """A top-K budget at least the number of pages selects, for every query
    page, all key pages up to its own (in ascending order), so the restricted
    attention is the full causal one ("Out of the Memory Barrier", section
    2.D, with the budget covering the context).  The sparse path then visits
    the same key tiles in the same order as the dense path: O, LSE and dQ must
    be bit-identical; dK/dV are the same sums, added by atomics in another
    order."""
    from paged_kv_cache_chunk_amd.chunks import Sparse

    n_ctx = 2000 if ragged else 2048
    cfg = mini_config("qwen_256k_topk", n_ctx=n_ctx, chunk=1024, top_k=16)
    w = Workload(cfg)
    dense = run_layer(cfg, w)
    sparse = run_layer(cfg, w, sparse=Sparse(top_k=cfg.n_pages))
    for c in range(cfg.n_chunks):
        pages, count = sparse["sel"][c]
        q_pos0, n = cfg.chunk_range(c)
        for il in range(pages.shape[0]):
            qpage = (q_pos0 + il * cfg.page) // cfg.page
            for g in range(cfg.hkv):
                assert list(pages[il, g, :count[il, g]]) == list(range(qpage + 1))
    for name in ("O", "lse", "dq"):
        assert np.array_equal(dense[name], sparse[name]), \
            f"{name}: max diff {np.abs(dense[name] - sparse[name]).max():.3e}"
    for name in ("dk", "dv"):
        assert rel_err(sparse[name], dense[name]) <= 1e-5, name
    dense["pool"].close()
    sparse["pool"].close()


@pytest.mark.parametrize("sparse_k", [0, 4])
def test_bf16_chunking_does_not_change_results(sparse_k):
    """Chunk-recurrent processing gives the results of the whole sequence
    whatever the (page-aligned) chunk size ("Out of the Memory Barrier",
    sections 2.A and 2.B): the same sequence cut into chunks of 512, 1024 and
    2048 rows.  A query row sees the same keys in the same tile order in every
    cut, so O, LSE and dQ are bit-identical; dK/dV collect the same
    contributions from a different number of chunks (fp32 atomics, another
    order).  In top-K mode a query page's selection depends only on its own
    rows and the keys before it, so the same holds."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from synthetic.gen import ChunkInputs

    base = mini_config("qwen_256k_topk", n_ctx=2048, chunk=2048, top_k=max(sparse_k, 1))
    w = Workload(base)
    f = w.full()  # one sequence, cut three ways below
    outs = []
    for chunk in (512, 1024, 2048):
        cfg = base.replace(chunk=chunk)
        cuts = [ChunkInputs(p0, f.q[p0:p0 + chunk], f.k[p0:p0 + chunk], f.v[p0:p0 + chunk],
                            f.do[p0:p0 + chunk]) for p0 in range(0, cfg.n_ctx, chunk)]
        sp = Sparse(top_k=sparse_k) if sparse_k else None
        outs.append(run_layer(cfg, w, sparse=sp, table=w.table(), chunks=cuts))
    ref = outs[-1]
    for got in outs[:-1]:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(got[name], ref[name]), \
                f"{name}: max diff {np.abs(got[name] - ref[name]).max():.3e}"
        for name in ("dk", "dv"):
            assert rel_err(got[name], ref[name]) <= 1e-5, name
    for o in outs:
        o["pool"].close()


@pytest.mark.parametrize("dtype,sparse_k", [("bf16", 0), ("bf16", 2), ("f32", 0)])
def test_single_token_context(dtype, sparse_k):
    """A context of one token.  The only row sees key 0 alone, so its one
    probability is 1: O is v0 (bit-exact in bf16, where any probability
    within 2^-9 of 1 rounds back to v0), LSE is the one scaled score, dV is
    dO summed over the group's query heads, and dQ, dK vanish ("Out of the
    Memory Barrier", section 2.A: dS = P (dP - D) with dP = D here) up to the
    rounding of two fp32 sums of the same d products, bounded below by
    1e-4 of the sum of their magnitudes.  In top-K mode the one query page
    selects page 0."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    base = "qwen_256k_topk" if sparse_k else "qwen_32k_dense"
    cfg = mini_config(base, n_ctx=1, chunk=128, top_k=sparse_k).replace(dtype=dtype)
    sp = Sparse(top_k=sparse_k) if sparse_k else None
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f = w.full()
    q, k, v, do = (x.astype(np.float64) for x in (f.q, f.k, f.v, f.do))
    G = cfg.group
    if sp is not None:
        pages, count = got["sel"][0]
        assert count.tolist() == [[1] * cfg.hkv]
        assert (pages[0, :, 0] == 0).all()
    for h in range(cfg.hq):
        g = h // G
        if dtype == "bf16":
            assert np.array_equal(got["O"][0, h], v[0, g]), h
        else:
            assert rel_err(got["O"][0, h], v[0, g]) <= 1e-6, h
        s = cfg.scale * float(q[0, h] @ k[0, g])
        assert abs(got["lse"][h, 0] - s) <= 1e-5 * max(1.0, abs(s)), h
        mag = cfg.scale * np.abs(do[0, h] * v[0, g]).sum() * np.abs(k[0, g]).max()
        assert np.abs(got["dq"][0, h]).max() <= 1e-4 * mag, h
    for g in range(cfg.hkv):
        heads = range(g * G, (g + 1) * G)
        assert rel_err(got["dv"][0, g], do[0, g * G:(g + 1) * G].sum(0)) <= TOL[dtype], g
        mag = cfg.scale * sum(np.abs(do[0, h] * v[0, g]).sum() * np.abs(q[0, h]).max()
                              for h in heads)
        assert np.abs(got["dk"][0, g]).max() <= 1e-4 * mag, g
    got["pool"].close()


@pytest.mark.parametrize("name,sparse_k", [("qwen_32k_dense", 0), ("qwen_256k_topk", 3),
                                           ("tiny_f32", 0)])
def test_one_token_last_chunk(name, sparse_k):
    """The last chunk is a single row that opens a new page after full pages:
    the shortest ragged tail (a one-row query tile, a one-key page and, in
    top-K mode, a one-row query page whose mean is that row)."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    if name == "tiny_f32":
        cfg = get_config(name).replace(n_ctx=513)
    else:
        cfg = mini_config(name, n_ctx=1025, chunk=512, top_k=sparse_k)
    assert cfg.chunk_range(cfg.n_chunks - 1)[1] == 1 and (cfg.n_ctx - 1) % cfg.page == 0
    sp = Sparse(top_k=sparse_k) if sparse_k else None
    w = Workload(cfg)
    got = run_layer(cfg, w, sparse=sp)
    f, ref = _oracle_for(cfg, w, sp)
    if sp is not None:
        ref = _check_sel(cfg, f, got, ref, sp)
    _check(cfg, got, ref, TOL[cfg.dtype])
    got["pool"].close()


@pytest.mark.parametrize("top_k", [1, 2, 4, 7])
def test_bf16_selection_ties_go_to_the_lower_page(top_k):
    """Exact ties on the GPU.  Key pages 4.. are copies of pages 1, 2 or 3, so
    the fp32 representatives of a template's copies are bit-identical (the
    same keys summed in the same order) and so are their scores: the budget
    cuts through groups of equal scores, where only the tie rule (the lower
    page index first) decides.  The scores of different templates lie at
    least 8e-5 apart on these seeded inputs (checked below on the oracle), far
    beyond any fp32 rounding difference, so the GPU's lists must equal the
    oracle's (fp32 scoring, ties to the lower page) exactly, with no gap
    allowance; then O, LSE, dQ, dK, dV against the oracle on that
    selection."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from synthetic.gen import ChunkInputs
    cfg = mini_config("qwen_256k_topk", n_ctx=3072, chunk=1024, top_k=top_k)
    w = Workload(cfg)
    f = w.full()
    P = cfg.page
    k = f.k.copy()
    for p in range(4, cfg.n_pages):
        t = 1 + (5 * p) % 3
        k[p * P:(p + 1) * P] = k[t * P:(t + 1) * P]
    chunks = []
    for c in range(cfg.n_chunks):
        q_pos0, n = cfg.chunk_range(c)
        sl = slice(q_pos0, q_pos0 + n)
        chunks.append(ChunkInputs(q_pos0, f.q[sl], k[sl], f.v[sl], f.do[sl]))
    sp = Sparse(top_k=top_k)
    got = run_layer(cfg, w, sparse=sp, chunks=chunks)
    ties_cut = 0
    for c in range(cfg.n_chunks):
        q_pos0, n = cfg.chunk_range(c)
        ref_sel = oracle.select_pages(f.q[q_pos0:q_pos0 + n], k, q_pos0, P, cfg.hkv, top_k,
                                      sp.n_sink, sp.n_local, score_dtype=np.float32)
        kbar = oracle.key_page_means(k[:q_pos0 + n], P).astype(np.float32)
        qbar = oracle.query_page_means(f.q[q_pos0:q_pos0 + n], P, cfg.hkv).astype(np.float32)
        for il, row in enumerate(sel_lists(got["sel"][c])):
            i = q_pos0 // P + il
            for g, lst in enumerate(row):
                assert lst == ref_sel[il][g].tolist(), (c, il, g, lst, ref_sel[il][g].tolist())
                cand = np.arange(sp.n_sink, i - sp.n_local + 1)
                if cand.size <= top_k:
                    continue
                s = np.sort((kbar[cand, g] * qbar[il, g][None]).sum(axis=1, dtype=np.float32))
                u = np.unique(s)
                assert u.size < 2 or np.diff(u).min() > 1e-5  # distinct scores well apart
                ties_cut += bool(s[::-1][top_k - 1] == s[::-1][top_k])
    assert ties_cut > 0, "no list had its budget cut through a tie"
    print(f"top_k {top_k}: {ties_cut} lists cut through a tie", flush=True)
    ref = oracle.run_chunks(f.q, k, f.v, f.do, cfg.chunk, cfg.scale, P, sels=_gpu_sels(cfg, got))
    _check(cfg, got, ref, TOL["bf16"])
    got["pool"].close()
