"""GPU: pkv_attn_bwd_noalloc (scratch in the library's fixed device array, no
allocation) gives the results of pkv_attn_bwd on the same inputs, on two
calls in a row, the second with a smaller chunk (the array keeps the first
call's contents), in dense and top-K mode, bf16 and fp32; a chunk whose
scratch exceeds the array is rejected with PKV_ECAPACITY before anything is
enqueued.  dQ is written by the same kernels, so it must be bit-identical;
dK/dV are fp32 atomic sums, equal up to the order of the adds.  Both are
also checked against the oracle."""
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


def _pair(cfg, calls, sparse_k):
    """Two layers holding the same K/V; each call (q_pos0, n_q) runs select +
    forward once, then the backward through pkv_attn_bwd on layer 0 and
    pkv_attn_bwd_noalloc on layer 1."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import Sparse, torch_dtype

    kvd = pkv.PKV_BF16 if cfg.dtype == "bf16" else pkv.PKV_F32
    dt = torch_dtype(kvd)
    w = Workload(cfg)
    f = w.full()
    pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, kvd)
    tab = w.table()
    for layer in (0, 1):
        for g in range(cfg.hkv):
            pkv.pkv_page_table_set(pool, layer, g, tab[g])
        pkv.pkv_append_kv(pool, layer, 0, torch.from_numpy(f.k).to(dt).cuda(),
                          torch.from_numpy(f.v).to(dt).cuda())
    sp = Sparse(sparse_k) if sparse_k else None
    sels = []
    for q_pos0, n in calls:
        print(f"call q_pos0={q_pos0} n_q={n} sparse_k={sparse_k} dtype={cfg.dtype}", flush=True)
        q = torch.from_numpy(f.q[q_pos0:q_pos0 + n]).to(dt).cuda()
        do = torch.from_numpy(f.do[q_pos0:q_pos0 + n]).to(dt).cuda()
        o = torch.empty_like(q)
        lse = torch.empty(cfg.hq, n, dtype=torch.float32, device="cuda")
        sel = None
        if sp is not None:
            nqp = -(-n // cfg.page)
            sel = (torch.empty(nqp, cfg.hkv, sp.stride, dtype=torch.int32, device="cuda"),
                   torch.empty(nqp, cfg.hkv, dtype=torch.int32, device="cuda"))
            pkv.pkv_select_topk_pages(pool, 0, q_pos0, q, sp.top_k, sel[0], sel[1])
        pkv.pkv_attn_fwd(pool, 0, q_pos0, q, o, lse, cfg.scale, sel=sel)
        dq0 = torch.full((n, cfg.hq, cfg.d), float("nan"), device="cuda")
        dq1 = torch.full((n, cfg.hq, cfg.d), float("nan"), device="cuda")
        pkv.pkv_attn_bwd(pool, 0, q_pos0, q, o, do, lse, dq0, cfg.scale, sel=sel)
        pkv.pkv_attn_bwd_noalloc(pool, 1, q_pos0, q, o, do, lse, dq1, cfg.scale, sel=sel)
        torch.cuda.synchronize()
        assert torch.equal(dq0, dq1), f"dQ differs (max {float((dq0 - dq1).abs().max()):.3e})"
        if sel is not None:
            pages, count = sel[0].cpu().numpy(), sel[1].cpu().numpy()
            sels.append([[pages[i, g, :count[i, g]].astype(np.int64) for g in range(cfg.hkv)]
                         for i in range(pages.shape[0])])
        else:
            sels.append(None)
        # each call's dQ against the oracle on that call's selection
        r = oracle.attn_bwd(f.q[q_pos0:q_pos0 + n], f.k, f.v, f.do[q_pos0:q_pos0 + n], q_pos0,
                            cfg.scale, cfg.page, sels[-1])
        tol = 1e-2 if cfg.dtype == "bf16" else 1e-5
        assert rel_err(dq1.cpu().numpy(), r["dq"]) <= tol
        # after each call the two layers' accumulated dK/dV agree
        got = []
        for layer in (0, 1):
            dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
            dv = torch.empty_like(dk)
            pkv.pkv_read_pages(pool, layer, pkv.PKV_DK, dk)
            pkv.pkv_read_pages(pool, layer, pkv.PKV_DV, dv)
            torch.cuda.synchronize()
            got.append((dk.cpu().numpy(), dv.cpu().numpy()))
        assert rel_err(got[1][0], got[0][0]) <= 1e-5
        assert rel_err(got[1][1], got[0][1]) <= 1e-5
    # accumulated over the calls: the oracle's sums
    dk_ref = np.zeros((cfg.n_ctx, cfg.hkv, cfg.d))
    dv_ref = np.zeros_like(dk_ref)
    for (q_pos0, n), sel in zip(calls, sels):
        r = oracle.attn_bwd(f.q[q_pos0:q_pos0 + n], f.k, f.v, f.do[q_pos0:q_pos0 + n], q_pos0,
                            cfg.scale, cfg.page, sel)
        dk_ref[:q_pos0 + n] += r["dk"]
        dv_ref[:q_pos0 + n] += r["dv"]
    tol = 1e-2 if cfg.dtype == "bf16" else 1e-5
    assert rel_err(got[1][0], dk_ref) <= tol
    assert rel_err(got[1][1], dv_ref) <= tol
    pool.close()


@pytest.mark.parametrize("sparse_k", [0, 3])
def test_noalloc_matches_bwd_bf16(sparse_k):
    base = "qwen_256k_topk" if sparse_k else "qwen_32k_dense"
    cfg = mini_config(base, n_ctx=2048, chunk=1024, top_k=max(sparse_k, 1))
    # the second call is smaller: 384 rows of the first pages
    _pair(cfg, [(768, 1280), (0, 384)], sparse_k)


def test_noalloc_matches_bwd_f32():
    cfg = get_config("tiny_f32")
    _pair(cfg, [(128, 384), (0, 96)], 0)


def test_noalloc_rejects_scratch_beyond_its_array():
    """2 x 28 heads x 75008 rows x 4 bytes = 16.8 MB of D and log-sum-exp:
    more than the 16 MiB array.  Every buffer has its full size, so nothing
    could be read out of bounds even if a kernel were launched."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    n = 75008
    pool = pkv.pkv_pool_create(1, 4, 128, 128, 600, 600, pkv.PKV_BF16)
    kv = torch.zeros(n, 4, 128, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append_kv(pool, 0, 0, kv, kv)
    q = torch.zeros(n, 28, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(28, n, device="cuda")
    dq = torch.zeros(n, 28, 128, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_bwd_noalloc(pool, 0, 0, q, q, q, lse, dq, 0.088)
    assert e.value.status == 3, str(e.value)  # PKV_ECAPACITY
    assert "scratch" in pkv.pkv_last_error()
    torch.cuda.synchronize()
    pool.close()
