"""GPU tests of the host tier: K/V and KV-gradient pools of several layers
in pinned host memory, a two-layer HBM window filled by pkv_prefetch_pages
on a side stream, gradient pages written back by pkv_writeback_grads
(or, with host_grad_accumulate, the window gradients zeroed instead of
fetched and each visit's contributions added into the host tier by the
library's host threads).

The offloaded sweep must give bit-identical O, LSE and dQ to the same sweep
on an all-HBM pool (same kernels, same K/V), and dK/dV within the bf16 bound
of the oracle (gradients round-trip through bf16 host pages) or within fp32
accumulation noise with an fp32 host gradient tier."""
import numpy as np
import pytest

import oracle
from synthetic import Workload, mini_config
from tests.gpu_util import compare_selection, gpu_available, rel_err, sel_lists

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


CFG = mini_config("qwen_1m_offload", n_ctx=4096, chunk=1024, n_layers=3, top_k=6,
                  slots=32)


def _sweep(cfg, host_tier, host_grad_dtype=None, sparse=True, accumulate=0, lookahead=False):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.chunks import ChunkBuffers, OffloadSweep, Sparse

    L = cfg.n_layers
    ws = [Workload(cfg, layer=l) for l in range(L)]
    chunks = {(l, c): ws[l].chunk(c) for l in range(L) for c in range(cfg.n_chunks)}
    pool = pkv.pkv_pool_create(L, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                               host_tier=int(host_tier),
                               host_grad_dtype=host_grad_dtype if host_grad_dtype is not None
                               else pkv.PKV_BF16,
                               device_budget_bytes=cfg.hbm_cap_bytes if host_tier else 0,
                               host_grad_accumulate=accumulate)
    for l in range(L):
        tab = ws[l].table()
        for g in range(cfg.hkv):
            pkv.pkv_page_table_set(pool, l, g, tab[g])
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    for c in range(cfg.n_chunks):          # forward sweep: appends, layer by layer
        for l in range(L):
            ch = chunks[(l, c)]
            pkv.pkv_append_kv(pool, l, ch.q_pos0, dev(ch.k), dev(ch.v))
    sp = Sparse(cfg.top_k, cfg.n_sink, cfg.n_local) if sparse else None
    sweep = OffloadSweep(pool, L, cfg.hq, cfg.hkv, cfg.d, cfg.page, cfg.scale, sp, torch.bfloat16)
    got = {}

    def inputs(l, c):
        ch = chunks[(l, c)]
        return dict(q_pos0=ch.q_pos0, q=dev(ch.q), do=dev(ch.do))

    def outputs(l, c, b):
        got[(l, c)] = dict(O=b.o.float().cpu(), lse=b.lse.cpu(), dq=b.dq.cpu(),
                           sel=(b.sel[0].cpu(), b.sel[1].cpu()) if sparse else None)

    def bufs_for(c):
        return {l: ChunkBuffers(chunks[(l, c)].n_q, cfg.hq, cfg.hkv, cfg.d, cfg.page,
                                torch.bfloat16, sp) for l in range(L)}

    order = list(reversed(range(cfg.n_chunks)))
    nxt = bufs_for(order[0])
    for i, c in enumerate(order):
        bufs, nxt = nxt, (bufs_for(order[i + 1]) if i + 1 < len(order) else None)
        # lookahead: the next chunk's top layer is prefetched during layer 0
        ahead = (order[i + 1], nxt) if lookahead and nxt is not None else None
        sweep.chunk(c, inputs, bufs, outputs, next_chunk=ahead)
    torch.cuda.synchronize()
    grads = {}
    for l in range(L):
        dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(pool, l, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, l, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        grads[l] = (dk.cpu().numpy(), dv.cpu().numpy())
    dev_b, host_b = pkv.pkv_pool_bytes(pool)
    moved = pkv.pkv_offload_bytes(pool)
    pool.close()
    return got, grads, chunks, (dev_b, host_b, moved)


def test_offloaded_matches_resident_and_oracle():
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG
    # three layers: the next chunk's top layer would share layer 0's window,
    # so the sweep must fall back to prefetching it at the chunk's start
    off, goff, chunks, (dev_b, host_b, _) = _sweep(cfg, True, lookahead=True)
    res, gres, _, (dev_r, host_r, _) = _sweep(cfg, False)
    # memory: the host tier holds every layer, HBM only the two-layer window
    assert host_b > 0 and host_r == 0
    assert dev_b < dev_r
    for key in res:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(off[key][name].numpy(), res[key][name].numpy()), (key, name)
        for x, y in zip(off[key]["sel"], res[key]["sel"]):
            assert np.array_equal(x.numpy(), y.numpy())
    for l in range(cfg.n_layers):
        w = Workload(cfg, layer=l)
        f = w.full()
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page,
                                sparse=dict(top_k=cfg.top_k, n_sink=cfg.n_sink,
                                            n_local=cfg.n_local, score_dtype=np.float32))
        for c in range(cfg.n_chunks):
            q_pos0, n = cfg.chunk_range(c)
            _, scores = oracle.select_pages(f.q[q_pos0:q_pos0 + n], f.k, q_pos0, cfg.page,
                                            cfg.hkv, cfg.top_k, cfg.n_sink, cfg.n_local,
                                            return_scores=True)
            nd = compare_selection(sel_lists(tuple(t.numpy() for t in off[(l, c)]["sel"])),
                                   ref["sel"][c], scores, cfg.top_k)
            assert nd == 0
            sl = slice(q_pos0, q_pos0 + n)
            assert rel_err(off[(l, c)]["O"].numpy(), ref["O"][sl]) < 1e-2
            assert rel_err(off[(l, c)]["dq"].numpy(), ref["dq"][sl]) < 1e-2
        e_off = max(rel_err(goff[l][0], ref["dk"]), rel_err(goff[l][1], ref["dv"]))
        e_res = max(rel_err(gres[l][0], ref["dk"]), rel_err(gres[l][1], ref["dv"]))
        print(f"layer {l}: dK/dV error, bf16 host grads {e_off:.2e}, all-HBM fp32 {e_res:.2e}",
              flush=True)
        assert e_off < 1e-2 and e_res < 1e-2


def test_offloaded_dense_matches_resident_and_oracle():
    """Dense chunks prefetch only the pages of keys up to their last query
    (pkv_prefetch_prefix) and write back the same pages' gradients."""
    cfg = CFG.replace(n_layers=2)
    off, goff, _, _ = _sweep(cfg, True, sparse=False, lookahead=True)
    res, gres, _, _ = _sweep(cfg, False, sparse=False)
    for key in res:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(off[key][name].numpy(), res[key][name].numpy()), (key, name)
    for l in range(cfg.n_layers):
        f = Workload(cfg, layer=l).full()
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page)
        for c in range(cfg.n_chunks):
            q_pos0, n = cfg.chunk_range(c)
            sl = slice(q_pos0, q_pos0 + n)
            assert rel_err(off[(l, c)]["O"].numpy(), ref["O"][sl]) < 1e-2
            assert rel_err(off[(l, c)]["dq"].numpy(), ref["dq"][sl]) < 1e-2
        e_off = max(rel_err(goff[l][0], ref["dk"]), rel_err(goff[l][1], ref["dv"]))
        e_res = max(rel_err(gres[l][0], ref["dk"]), rel_err(gres[l][1], ref["dv"]))
        print(f"dense layer {l}: dK/dV error, bf16 host grads {e_off:.2e}, all-HBM fp32 {e_res:.2e}",
              flush=True)
        assert e_off < 1e-2 and e_res < 1e-2


def test_prefetch_prefix_arguments():
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                               pkv.PKV_BF16, host_tier=1)
    k = torch.zeros(256, cfg.hkv, cfg.d, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append_kv(pool, 0, 0, k, k)
    for bad in (0, 257):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_prefetch_prefix(pool, 0, bad)
        assert e.value.status == 1  # PKV_EINVAL
    with pytest.raises(pkv.PkvError):
        pkv.pkv_prefetch_prefix(pool, 2, 1)
    pkv.pkv_prefetch_prefix(pool, 0, 256, with_grads=True)
    torch.cuda.synchronize()
    pool.close()


def test_offloaded_fp32_grad_tier_matches_resident():
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    _, goff, _, _ = _sweep(cfg, True, pkv.PKV_F32)
    _, gres, _, _ = _sweep(cfg, False)
    for l in range(cfg.n_layers):
        assert rel_err(goff[l][0], gres[l][0]) < 1e-5
        assert rel_err(goff[l][1], gres[l][1]) < 1e-5


def test_attention_before_prefetch_is_an_error():
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                               pkv.PKV_BF16, host_tier=1)
    k = torch.zeros(256, cfg.hkv, cfg.d, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append_kv(pool, 1, 0, k, k)
    q = torch.zeros(256, cfg.hq, cfg.d, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, 256, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_fwd(pool, 1, 0, q, o, lse, cfg.scale)
    assert e.value.status == 4  # PKV_ESTATE
    pkv.pkv_prefetch_pages(pool, 1)
    pkv.pkv_attn_fwd(pool, 1, 0, q, o, lse, cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    pool.close()


@pytest.mark.parametrize("sparse", [True, False])
def test_host_accumulated_grads_match_oracle(sparse):
    """host_grad_accumulate: same O, LSE, dQ and selections as the all-HBM
    sweep; dK/dV within the bf16 bound of the oracle (contribution and sum
    are each rounded to bf16 per visit); no gradient bytes fetched.  Both
    offloaded sweeps prefetch the next chunk's top layer during layer 0."""
    cfg = CFG.replace(n_layers=2)
    off, goff, _, (_, host_a, (fetched_a, written_a)) = _sweep(cfg, True, sparse=sparse, accumulate=1,
                                                               lookahead=True)
    _, gfetch, _, (_, host_f, (fetched_f, written_f)) = _sweep(cfg, True, sparse=sparse,
                                                               lookahead=True)
    res, _, _, _ = _sweep(cfg, False, sparse=sparse)
    for key in res:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(off[key][name].numpy(), res[key][name].numpy()), (key, name)
        if sparse:
            for x, y in zip(off[key]["sel"], res[key]["sel"]):
                assert np.array_equal(x.numpy(), y.numpy())
    # the same pages move; host -> HBM carries K/V only (as many bytes as the
    # bf16 gradients it no longer carries), HBM -> host the same bytes as before
    assert written_a == written_f
    assert fetched_a * 2 == fetched_f
    assert host_a > host_f  # the pinned staging
    sp = dict(top_k=cfg.top_k, n_sink=cfg.n_sink, n_local=cfg.n_local,
              score_dtype=np.float32) if sparse else None
    for l in range(cfg.n_layers):
        f = Workload(cfg, layer=l).full()
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page, sparse=sp)
        e_acc = max(rel_err(goff[l][0], ref["dk"]), rel_err(goff[l][1], ref["dv"]))
        e_fetch = max(rel_err(gfetch[l][0], ref["dk"]), rel_err(gfetch[l][1], ref["dv"]))
        print(f"layer {l} sparse={sparse}: dK/dV error, host adds {e_acc:.2e}, "
              f"device adds {e_fetch:.2e}", flush=True)
        assert e_acc < 1e-2 and e_fetch < 1e-2


def test_host_accumulated_fp32_grad_tier_matches_resident():
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    _, goff, _, _ = _sweep(cfg, True, pkv.PKV_F32, accumulate=1)
    _, gres, _, _ = _sweep(cfg, False)
    for l in range(cfg.n_layers):
        assert rel_err(goff[l][0], gres[l][0]) < 1e-5
        assert rel_err(goff[l][1], gres[l][1]) < 1e-5


def test_host_accumulate_state_errors():
    """A second writeback of one prefetch would add the same contributions
    twice: PKV_ESTATE.  host_grad_accumulate without a host tier: PKV_EINVAL."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                            host_grad_accumulate=1)
    assert e.value.status == 1  # PKV_EINVAL
    pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                               pkv.PKV_BF16, host_tier=1, host_grad_accumulate=1)
    k = torch.ones(256, cfg.hkv, cfg.d, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append_kv(pool, 0, 0, k, k)
    pkv.pkv_prefetch_prefix(pool, 0, 256, with_grads=True)
    pkv.pkv_writeback_grads(pool, 0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_writeback_grads(pool, 0)
    assert e.value.status == 4  # PKV_ESTATE
    pkv.pkv_prefetch_prefix(pool, 0, 256, with_grads=True)
    pkv.pkv_writeback_grads(pool, 0)
    dk = torch.empty(256, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
    torch.cuda.synchronize()
    assert int((dk != 0).sum()) == 0  # nothing was computed: the adds added zeros
    pool.close()
