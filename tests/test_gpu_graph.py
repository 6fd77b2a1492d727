"""GPU: one chunk's attention calls captured in a HIP graph (torch.cuda.graph):
top-K selection, forward and the no-allocation backward (the entry point for
callers that cannot allocate, such as code under graph capture; its scratch
is the library's fixed device array and it records no memset).  The graph is
replayed several times; before each replay the program does eager work of
its own (dK/dV zeroed through pkv_grad_zero, the outputs overwritten, a torch
product) and synchronises, and every replay is checked against the same
calls made eagerly: the selection, O, LSE and dQ bit-identical (the same
kernels on the same inputs), dK/dV equal up to the order of the fp32 atomic
adds.  dQ of the eager run is also checked against the oracle."""
import numpy as np
import pytest

import oracle
from synthetic import Workload, get_config, mini_config
from tests.gpu_util import gpu_available, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


CASES = {
    # ragged last chunk (200 rows, a partial page) of a Qwen-shaped layer
    "bf16_dense": (lambda: mini_config("qwen_32k_dense", n_ctx=2 * 1024 + 200, chunk=1024), 0),
    "bf16_topk": (lambda: mini_config("qwen_256k_topk", n_ctx=5 * 1024 + 200, chunk=1024,
                                      top_k=4), 4),
    "f32_topk": (lambda: get_config("tiny_f32"), 2),
    # a last chunk of 28 query blocks x 28 heads: on a 256-CU device the
    # forward splits its last pass of workgroups and adds a merge kernel
    "bf16_topk_split": (lambda: mini_config("qwen_256k_topk", n_ctx=2 * 3584, chunk=3584,
                                            top_k=6), 6),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager_calls(case):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import Sparse, torch_dtype

    make_cfg, sparse_k = CASES[case]
    cfg = make_cfg()
    kvd = pkv.PKV_BF16 if cfg.dtype == "bf16" else pkv.PKV_F32
    dt = torch_dtype(kvd)
    w = Workload(cfg)
    f = w.full()
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, kvd)
    tab = w.table()
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    pkv.pkv_append_kv(pool, 0, 0, torch.from_numpy(f.k).to(dt).cuda(),
                      torch.from_numpy(f.v).to(dt).cuda())
    q_pos0, n = cfg.chunk_range(cfg.n_chunks - 1)
    print(f"{case}: q_pos0={q_pos0} n_q={n} sparse_k={sparse_k}", flush=True)
    q = torch.from_numpy(f.q[q_pos0:]).to(dt).cuda()
    do = torch.from_numpy(f.do[q_pos0:]).to(dt).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, n, dtype=torch.float32, device="cuda")
    dq = torch.empty(n, cfg.hq, cfg.d, dtype=torch.float32, device="cuda")
    sp = Sparse(sparse_k) if sparse_k else None
    sel = None
    if sp is not None:
        nqp = -(-n // cfg.page)
        sel = (torch.empty(nqp, cfg.hkv, sp.stride, dtype=torch.int32, device="cuda"),
               torch.empty(nqp, cfg.hkv, dtype=torch.int32, device="cuda"))

    def calls():
        if sp is not None:
            pkv.pkv_select_topk_pages(pool, 0, q_pos0, q, sp.top_k, sel[0], sel[1],
                                      sp.n_sink, sp.n_local)
        pkv.pkv_attn_fwd(pool, 0, q_pos0, q, o, lse, cfg.scale, sel=sel)
        pkv.pkv_attn_bwd_noalloc(pool, 0, q_pos0, q, o, do, lse, dq, cfg.scale, sel=sel)

    def grads():
        dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        return dk.cpu().numpy(), dv.cpu().numpy()

    def outputs():
        out = dict(o=o.clone(), lse=lse.clone(), dq=dq.clone())
        if sel is not None:
            out["pages"], out["count"] = sel[0].clone(), sel[1].clone()
        return out

    def poison():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        dq.fill_(float("nan"))
        if sel is not None:
            sel[0].fill_(-7)
            sel[1].fill_(-7)

    # eager reference (this call also sizes the selection's scratch and the
    # forward's split scratch, so that nothing grows under capture)
    pkv.pkv_grad_zero(pool, 0)
    poison()
    calls()
    torch.cuda.synchronize()
    ref = outputs()
    ref_dk, ref_dv = grads()
    sels = None
    if sel is not None:
        pages, count = ref["pages"].cpu().numpy(), ref["count"].cpu().numpy()
        sels = [[pages[i, g, :count[i, g]].astype(np.int64) for g in range(cfg.hkv)]
                for i in range(pages.shape[0])]
    r = oracle.attn_bwd(f.q[q_pos0:], f.k, f.v, f.do[q_pos0:], q_pos0, cfg.scale, cfg.page, sels)
    tol = 1e-2 if cfg.dtype == "bf16" else 1e-5
    assert rel_err(ref["dq"].cpu().numpy(), r["dq"]) <= tol
    assert rel_err(ref_dk[:q_pos0 + n], r["dk"]) <= tol
    assert rel_err(ref_dv[:q_pos0 + n], r["dv"]) <= tol

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        pkv.pkv_grad_zero(pool, 0)
        poison()
        a = torch.tanh(a @ a.T / 512.0)  # the program's own work between replays
        torch.cuda.synchronize()
        print(f"{case}: replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, t in ref.items():
            assert torch.equal(got[name], t), (case, rep, name)
        dk, dv = grads()
        assert rel_err(dk, ref_dk) <= 1e-5, (case, rep)
        assert rel_err(dv, ref_dv) <= 1e-5, (case, rep)
    del graph
    pool.close()
