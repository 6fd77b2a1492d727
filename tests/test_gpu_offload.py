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


def _sweep(cfg, host_tier, host_grad_dtype=None, sparse=True, accumulate=0, lookahead=False,
           window_slots=0, select_ahead=False):
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
                               host_grad_accumulate=accumulate,
                               window_slots=window_slots if host_tier else 0)
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
    if select_ahead and sp is not None:
        sweep.select_all(range(L), order, inputs)
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
        gpu_sels = []
        for c in range(cfg.n_chunks):
            q_pos0, n = cfg.chunk_range(c)
            ref_sel, scores = oracle.select_pages(f.q[q_pos0:q_pos0 + n], f.k, q_pos0, cfg.page,
                                                  cfg.hkv, cfg.top_k, cfg.n_sink, cfg.n_local,
                                                  score_dtype=np.float32, return_scores=True)
            gsel = sel_lists(tuple(t.numpy() for t in off[(l, c)]["sel"]))
            compare_selection(gsel, ref_sel, scores, cfg.top_k)  # gap rule, asserted inside
            gpu_sels.append([[np.array(x, dtype=np.int64) for x in row] for row in gsel])
        # values on the GPU's selections (which the gap rule admits)
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page,
                                sels=gpu_sels)
        for c in range(cfg.n_chunks):
            q_pos0, n = cfg.chunk_range(c)
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
    for bad in (0, cfg.n_pages * cfg.page + 1):
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


@pytest.mark.parametrize("accumulate", [0, 1])
def test_failed_transfers_leave_a_consistent_pool(accumulate):
    """A prefetch or a writeback whose copy fails to enqueue (forced through
    the library's test hook PKV_FAIL_COPY_AT=n: the n-th host-link copy of
    the pool, counted while the variable is set, fails as a failed launch
    would) returns PKV_EHIP.  After the failed prefetch the window holds no
    layer, so attention on it is PKV_ESTATE instead of reading pages that
    were never fetched; after the failed writeback the window's gradients
    stay in place.  Retrying both gives what a run without failures gives:
    O, LSE and dQ bit-identical, dK/dV within fp32 summation-order noise
    (fp32 host gradients)."""
    import os
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    w = Workload(cfg, layer=1)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    last = w.chunk(cfg.n_chunks - 1)
    n_keys = last.q_pos0 + last.n_q

    def run(fail):
        pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                                   pkv.PKV_BF16, host_tier=1, host_grad_dtype=pkv.PKV_F32,
                                   host_grad_accumulate=accumulate)
        tab = w.table()
        for g in range(cfg.hkv):
            pkv.pkv_page_table_set(pool, 1, g, tab[g])
        for c in range(cfg.n_chunks):
            ch = w.chunk(c)
            pkv.pkv_append_kv(pool, 1, ch.q_pos0, dev(ch.k), dev(ch.v))
        q, do = dev(last.q), dev(last.do)
        o = torch.empty_like(q)
        lse = torch.empty(cfg.hq, last.n_q, device="cuda")
        dq = torch.empty(last.n_q, cfg.hq, cfg.d, device="cuda")
        if fail:
            os.environ["PKV_FAIL_COPY_AT"] = "1"      # the pool's first copy: this fetch
            try:
                with pytest.raises(pkv.PkvError) as e:
                    pkv.pkv_prefetch_prefix(pool, 1, n_keys, with_grads=True)
            finally:
                del os.environ["PKV_FAIL_COPY_AT"]
            assert e.value.status == 5 and "injected" in str(e.value), str(e.value)
            with pytest.raises(pkv.PkvError) as e:
                pkv.pkv_attn_fwd(pool, 1, last.q_pos0, q, o, lse, cfg.scale)
            assert e.value.status == 4  # PKV_ESTATE: the window holds no layer
        pkv.pkv_prefetch_prefix(pool, 1, n_keys, with_grads=True)
        pkv.pkv_attn_fwd(pool, 1, last.q_pos0, q, o, lse, cfg.scale)
        pkv.pkv_attn_bwd(pool, 1, last.q_pos0, q, o, do, lse, dq, cfg.scale)
        if fail:
            os.environ["PKV_FAIL_COPY_AT"] = "2"      # the next copy counted: this writeback
            try:
                with pytest.raises(pkv.PkvError) as e:
                    pkv.pkv_writeback_grads(pool, 1)
            finally:
                del os.environ["PKV_FAIL_COPY_AT"]
            assert e.value.status == 5 and "injected" in str(e.value), str(e.value)
        pkv.pkv_writeback_grads(pool, 1)
        dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(pool, 1, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, 1, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        out = dict(O=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.cpu().numpy(),
                   dk=dk.cpu().numpy(), dv=dv.cpu().numpy())
        pool.close()
        return out

    ok, failed = run(False), run(True)
    for name in ("O", "lse", "dq"):
        assert np.array_equal(failed[name], ok[name]), name
    for name in ("dk", "dv"):
        assert np.abs(ok[name]).max() > 0
        assert rel_err(failed[name], ok[name]) < 1e-5, name


@pytest.mark.parametrize("accumulate", [0, 1])
def test_copy_streams_and_grad_zero_are_ordered(accumulate):
    """Two prefetches into one window slot issued on two different copy
    streams (layers 0 and 2 share window 0; the first prefetch is never
    used): the second waits for the first's copies, so the window ends up
    holding layer 2 alone and attention on it gives what the same calls on
    one copy stream give (O, LSE, dQ bit-identical; dK/dV within fp32
    summation-order noise, fp32 host gradients).  Then a writeback on one
    copy stream followed at once by pkv_grad_zero on another: the zeroing
    waits for the writeback (and the host adds), so the layer's gradients
    read back as zeros."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG  # 3 layers
    ws = {l: Workload(cfg, layer=l) for l in (0, 2)}
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    last = ws[2].chunk(cfg.n_chunks - 1)
    n_keys = last.q_pos0 + last.n_q

    def run(two_streams):
        pool = pkv.pkv_pool_create(3, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots,
                                   pkv.PKV_BF16, host_tier=1, host_grad_dtype=pkv.PKV_F32,
                                   host_grad_accumulate=accumulate)
        for l, w in ws.items():
            tab = w.table()
            for g in range(cfg.hkv):
                pkv.pkv_page_table_set(pool, l, g, tab[g])
            for c in range(cfg.n_chunks):
                ch = w.chunk(c)
                pkv.pkv_append_kv(pool, l, ch.q_pos0, dev(ch.k), dev(ch.v))
        torch.cuda.synchronize()
        s1 = torch.cuda.Stream()
        s2 = torch.cuda.Stream() if two_streams else s1
        q, do = dev(last.q), dev(last.do)
        o = torch.empty_like(q)
        lse = torch.empty(cfg.hq, last.n_q, device="cuda")
        dq = torch.empty(last.n_q, cfg.hq, cfg.d, device="cuda")
        pkv.pkv_prefetch_pages(pool, 0, None, with_grads=True, copy_stream=s1)
        pkv.pkv_prefetch_prefix(pool, 2, n_keys, with_grads=True, copy_stream=s2)
        pkv.pkv_attn_fwd(pool, 2, last.q_pos0, q, o, lse, cfg.scale)
        pkv.pkv_attn_bwd(pool, 2, last.q_pos0, q, o, do, lse, dq, cfg.scale)
        pkv.pkv_writeback_grads(pool, 2, copy_stream=s1)
        dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        pkv.pkv_read_pages(pool, 2, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, 2, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        out = dict(O=o.float().cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.cpu().numpy(),
                   dk=dk.cpu().numpy(), dv=dv.cpu().numpy())
        # a second visit's writeback, then the zeroing on the other stream
        pkv.pkv_prefetch_prefix(pool, 2, n_keys, with_grads=True, copy_stream=s2)
        pkv.pkv_attn_bwd(pool, 2, last.q_pos0, q, o, do, lse, dq, cfg.scale)
        pkv.pkv_writeback_grads(pool, 2, copy_stream=s1)
        pkv.pkv_grad_zero(pool, 2, stream=s2)
        pkv.pkv_read_pages(pool, 2, pkv.PKV_DK, dk)
        pkv.pkv_read_pages(pool, 2, pkv.PKV_DV, dv)
        torch.cuda.synchronize()
        out["zeroed"] = float(max(dk.abs().max().item(), dv.abs().max().item()))
        pool.close()
        return out

    one, two = run(False), run(True)
    for name in ("O", "lse", "dq"):
        assert np.array_equal(two[name], one[name]), name
    for name in ("dk", "dv"):
        assert np.abs(one[name]).max() > 0
        assert rel_err(two[name], one[name]) < 1e-5, name
    assert one["zeroed"] == 0.0 and two["zeroed"] == 0.0


# 64 pages per layer, chunks of 4 query pages, top-K 6 + 3 forced: a visit
# names at most 4 x 9 = 36 pages per KV head, so a window of 36 slots per head
# holds any selection while a layer has 64 pages
SMALL = mini_config("qwen_1m_offload", n_ctx=8192, chunk=512, n_layers=2, top_k=6, slots=64)


def test_host_adds_without_room_for_the_device_staging():
    """Host adds with a device budget that holds the windows but not the
    writeback's device staging: the pool is created without it (the writeback
    kernel writes the pinned staging itself, indexed like the tier), its
    device bytes are exactly the staging's fewer, and the sweep gives the
    staged sweep's results: O, LSE, dQ and the selections bit-identical, dK/dV
    within the bf16 bound of the staged sweep's and of the oracle."""
    cfg = CFG
    staged, g_staged, _, (dev_s, _, moved_s) = _sweep(cfg, True, accumulate=1, lookahead=True)
    stage = 2 * cfg.hkv * cfg.n_pages * cfg.page * cfg.d * 2  # dK, dV of a window, bf16
    tight = cfg.replace(hbm_cap_bytes=dev_s - stage)
    plain, g_plain, _, (dev_p, _, moved_p) = _sweep(tight, True, accumulate=1, lookahead=True)
    assert dev_p == dev_s - stage
    assert moved_p == moved_s
    for key in staged:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(plain[key][name].numpy(), staged[key][name].numpy()), (key, name)
        for x, y in zip(plain[key]["sel"], staged[key]["sel"]):
            assert np.array_equal(x.numpy(), y.numpy())
    for l in range(cfg.n_layers):
        f = Workload(cfg, layer=l).full()
        sels = [[[np.asarray(staged[(l, c)]["sel"][0][i, g, :staged[(l, c)]["sel"][1][i, g]]
                  .numpy(), dtype=np.int64) for g in range(cfg.hkv)]
                 for i in range(staged[(l, c)]["sel"][0].shape[0])] for c in range(cfg.n_chunks)]
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page, sels=sels)
        for which, i in (("dk", 0), ("dv", 1)):
            e_pair = rel_err(g_plain[l][i], g_staged[l][i])
            e_ref = rel_err(g_plain[l][i], ref[which])
            print(f"layer {l} {which}: unstaged vs staged {e_pair:.2e}, vs oracle {e_ref:.2e}",
                  flush=True)
            assert e_pair < 1e-2 and e_ref < 1e-2


@pytest.mark.parametrize("accumulate", [0, 1])
def test_small_window_matches_resident_and_oracle(accumulate):
    """Windows of 36 slots per KV head for layers of 64 pages: each visit packs
    its pages into the window's first slots and the kernels reach them through
    the window's table.  O, LSE, dQ and the selections must be bit-identical
    to the all-HBM sweep, dK/dV within the bf16 bound of the oracle, and the
    device bytes those of the smaller windows (with host adds, and of the
    smaller writeback staging)."""
    cfg = SMALL
    off, goff, _, (dev_s, _, moved_s) = _sweep(cfg, True, accumulate=accumulate, lookahead=True,
                                               window_slots=36)
    _, _, _, (dev_w, _, moved_w) = _sweep(cfg, True, accumulate=accumulate, lookahead=True)
    res, gres, _, _ = _sweep(cfg, False)
    for key in res:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(off[key][name].numpy(), res[key][name].numpy()), (key, name)
        for x, y in zip(off[key]["sel"], res[key]["sel"]):
            assert np.array_equal(x.numpy(), y.numpy())
    # the same pages move, in windows of 36 instead of 64 slots per head
    assert moved_s == moved_w
    page_head = cfg.page * cfg.d
    # host adds: the writeback's device staging (dK and dV of a window's
    # page-heads, bf16) shrinks with the window too
    stage = 2 * cfg.hkv * (64 - 36) * page_head * 2 if accumulate else 0
    assert dev_w - dev_s == 2 * cfg.hkv * (64 - 36) * page_head * (2 * 2 + 2 * 4) + \
        8 * 2 * 2 * cfg.hkv * (64 - 36) + stage
    for l in range(cfg.n_layers):
        f = Workload(cfg, layer=l).full()
        sels = [[[np.asarray(off[(l, c)]["sel"][0][i, g, :off[(l, c)]["sel"][1][i, g]]
                  .numpy(), dtype=np.int64) for g in range(cfg.hkv)]
                 for i in range(off[(l, c)]["sel"][0].shape[0])] for c in range(cfg.n_chunks)]
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page, sels=sels)
        e_off = max(rel_err(goff[l][0], ref["dk"]), rel_err(goff[l][1], ref["dv"]))
        e_res = max(rel_err(gres[l][0], ref["dk"]), rel_err(gres[l][1], ref["dv"]))
        print(f"layer {l} window 36 accumulate={accumulate}: dK/dV error {e_off:.2e} "
              f"(all-HBM {e_res:.2e})", flush=True)
        assert e_off < 1e-2 and e_res < 1e-2


def test_window_capacity_and_visit_state_errors():
    """A prefetch whose pages could exceed the window: PKV_ECAPACITY, nothing
    enqueued.  Tokens appended after a prefetch are not in the window:
    attention on them is PKV_ESTATE until the next prefetch, attention on the
    keys it holds still runs and matches the oracle.  A backward after a
    prefetch without gradients: PKV_ESTATE."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = SMALL
    w = Workload(cfg)
    f = w.full()
    pool = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                               host_tier=1, window_slots=36)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    pkv.pkv_append_kv(pool, 0, 0, dev(f.k[:4096]), dev(f.v[:4096]))   # 32 pages
    with pytest.raises(pkv.PkvError) as e:                            # 37 pages > 36
        pkv.pkv_append_kv(pool, 0, 4096, dev(f.k[4096:4736]), dev(f.v[4096:4736]))
        pkv.pkv_prefetch_prefix(pool, 0, 4736)
    assert e.value.status == 3, str(e.value)  # PKV_ECAPACITY
    # dense prefetch of 4096 keys (32 pages), then more tokens are appended
    pkv.pkv_pool_reset(pool, 0)
    pkv.pkv_append_kv(pool, 0, 0, dev(f.k[:4096]), dev(f.v[:4096]))
    pkv.pkv_prefetch_prefix(pool, 0, 4096, with_grads=True)
    pkv.pkv_append_kv(pool, 0, 4096, dev(f.k[4096:4224]), dev(f.v[4096:4224]))
    q_pos0, n = 3584, 640
    q = dev(f.q[q_pos0:q_pos0 + n])
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, n, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_fwd(pool, 0, q_pos0, q, o, lse, cfg.scale)
    assert e.value.status == 4, str(e.value)  # PKV_ESTATE: rows 4096.. are not in the window
    # the rows the window covers still run
    n = 512
    q, do = dev(f.q[q_pos0:q_pos0 + n]), dev(f.do[q_pos0:q_pos0 + n])
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, n, device="cuda")
    dq = torch.empty(n, cfg.hq, cfg.d, device="cuda")
    pkv.pkv_attn_fwd(pool, 0, q_pos0, q, o, lse, cfg.scale)
    pkv.pkv_attn_bwd(pool, 0, q_pos0, q, o, do, lse, dq, cfg.scale)
    torch.cuda.synchronize()
    r = oracle.attn_bwd(f.q[q_pos0:q_pos0 + n], f.k, f.v, f.do[q_pos0:q_pos0 + n], q_pos0,
                        cfg.scale, cfg.page)
    assert rel_err(o.float().cpu().numpy(), r["O"]) < 1e-2
    assert rel_err(dq.cpu().numpy(), r["dq"]) < 1e-2
    pkv.pkv_writeback_grads(pool, 0)
    # layer 1: K/V only, then a backward
    pkv.pkv_append_kv(pool, 1, 0, dev(f.k[:1024]), dev(f.v[:1024]))
    pkv.pkv_prefetch_prefix(pool, 1, 1024, with_grads=False)
    q, do = dev(f.q[:512]), dev(f.do[:512])
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, 512, device="cuda")
    dq = torch.empty(512, cfg.hq, cfg.d, device="cuda")
    pkv.pkv_attn_fwd(pool, 1, 0, q, o, lse, cfg.scale)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_bwd(pool, 1, 0, q, o, do, lse, dq, cfg.scale)
    assert e.value.status == 4, str(e.value)
    torch.cuda.synchronize()
    pool.close()


def test_pool_bytes_are_the_page_bytes():
    """The pools hold exactly their page bytes: K, V (kv dtype) and dK, dV
    (fp32) per slot, one fp32 representative per slot and the int32 page
    tables (sciencestack.ai, Figure 4: a store that is not paged costs about
    three times the theoretical memory).  Host tier: the tier holds every
    layer's pages (gradients in the host dtype); HBM the two windows, their
    tables, page maps and lists, and two byte counters."""
    import paged_kv_cache_chunk_amd as pkv
    L, hkv, d, P, pages, slots = 3, 4, 128, 128, 40, 48
    page_head = P * d
    reps_tab = L * hkv * slots * d * 4 + L * hkv * pages * 4
    pool = pkv.pkv_pool_create(L, hkv, d, P, pages, slots, pkv.PKV_BF16)
    dev_b, host_b = pkv.pkv_pool_bytes(pool)
    pool.close()
    assert host_b == 0
    assert dev_b == L * hkv * slots * page_head * (2 + 2 + 4 + 4) + reps_tab
    pool = pkv.pkv_pool_create(1, 1, 64, 16, 32, 40, pkv.PKV_F32)
    dev_b, _ = pkv.pkv_pool_bytes(pool)
    pool.close()
    assert dev_b == 40 * 16 * 64 * 16 + 40 * 64 * 4 + 32 * 4
    for ws in (0, 24):
        wsl = ws or pages
        pool = pkv.pkv_pool_create(L, hkv, d, P, pages, slots, pkv.PKV_BF16, host_tier=1,
                                   window_slots=ws)
        dev_b, host_b = pkv.pkv_pool_bytes(pool)
        pool.close()
        assert host_b == L * hkv * slots * page_head * (2 + 2 + 2 + 2)
        assert dev_b == (2 * hkv * wsl * page_head * (2 + 2 + 4 + 4) + reps_tab
                         + 2 * hkv * pages * 4          # window tables
                         + 2 * 2 * hkv * pages          # page maps
                         + 8 * 2 * 2 * hkv * wsl        # page-head lists
                         + 4 * 2 * 2 + 16)              # list lengths, byte counters


def test_two_million_token_pool_fits_the_hbm_cap():
    """2M tokens (16384 pages per KV head) with host-tier pools and windows of
    64 x 131 = 8384 slots per head, what a chunk of 8192 tokens with top-K
    128 + 3 forced pages can name: creation succeeds under the 16 GiB cap, and
    the device bytes grow with the context only by the representatives and
    page tables (two layers here: the box pins at most 64 GiB per process)."""
    import paged_kv_cache_chunk_amd as pkv
    hkv, d, P, ws = 4, 128, 128, 64 * 131
    sizes = {}
    for n_pages in (4096, 8192, 16384):
        pool = pkv.pkv_pool_create(2, hkv, d, P, n_pages, n_pages, pkv.PKV_BF16, host_tier=1,
                                   window_slots=ws, device_budget_bytes=16 << 30)
        sizes[n_pages] = pkv.pkv_pool_bytes(pool)[0]
        pool.close()
    print({k * P: v for k, v in sizes.items()}, flush=True)
    for n, got in sizes.items():
        w = min(ws, n)  # a window never holds more than a layer
        assert got == (2 * hkv * w * P * d * (2 + 2 + 4 + 4)   # two windows
                       + 2 * hkv * n * (d * 4 + 4)             # reps, page tables (2 layers)
                       + 2 * hkv * n * 4 + 2 * 2 * hkv * n     # window tables, page maps
                       + 8 * 2 * 2 * hkv * w + 32)             # lists, lengths, counters
    # beyond the window's size the context costs only the per-page metadata
    assert sizes[16384] - sizes[8192] == (2 * hkv * (8384 - 8192) * P * d * 12
                                          + 8192 * 2 * hkv * (d * 4 + 4 + 4 + 2)
                                          + 8 * 4 * hkv * (8384 - 8192))
    assert sizes[16384] < 16 << 30


# 16K tokens in 128 chunks of one page, top-K 8 + 3 forced pages: the sink
# page is in every chunk's selection (128 visits), planted pages in many.
MANY = mini_config("qwen_1m_offload", n_ctx=16384, chunk=128, n_layers=2, top_k=8, slots=128,
                   hq=4, hkv=1)


def test_many_visit_gradient_accumulation():
    """Gradients accumulated over up to 128 visits of a page, against the
    oracle for every dK/dV element: the all-HBM pool (fp32 atomics in place),
    the bf16 host tier with gradients fetched and written back each visit
    (one bf16 rounding of the running sum per visit), the bf16 host tier with
    host-side adds (the visit's contribution and the sum rounded per visit),
    and the fp32 host tier (no rounding; within 1e-5 of the all-HBM pool).
    Prints the error of each tier by the number of visits of the page."""
    import paged_kv_cache_chunk_amd as pkv
    cfg = MANY
    runs = {
        "all-HBM": _sweep(cfg, False),
        "bf16 tier": _sweep(cfg, True, lookahead=True),
        "bf16 tier, host adds": _sweep(cfg, True, accumulate=1, lookahead=True),
        "fp32 tier": _sweep(cfg, True, pkv.PKV_F32, lookahead=True),
    }
    base = runs["all-HBM"][0]
    for name, (got, _, _, _) in runs.items():
        for key in base:
            for t in ("O", "lse", "dq"):
                assert np.array_equal(got[key][t].numpy(), base[key][t].numpy()), (name, key, t)
    P = cfg.page
    for l in range(cfg.n_layers):
        f = Workload(cfg, layer=l).full()
        sels, visits = [], np.zeros(cfg.n_pages, dtype=np.int64)
        for c in range(cfg.n_chunks):
            pages, count = (t.numpy() for t in base[(l, c)]["sel"])
            lst = pages[0, 0, :count[0, 0]].astype(np.int64)
            sels.append([[lst]])
            visits[lst] += 1
        q_pos0, n = cfg.chunk_range(cfg.n_chunks - 1)
        ref_sel, scores = oracle.select_pages(f.q[q_pos0:], f.k, q_pos0, P, cfg.hkv, cfg.top_k,
                                              cfg.n_sink, cfg.n_local, score_dtype=np.float32,
                                              return_scores=True)
        compare_selection([[sels[-1][0][0].tolist()]], ref_sel, scores, cfg.top_k)
        ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, P, sels=sels)
        assert visits.max() == cfg.n_chunks  # the sink page: every chunk
        vis_tok = np.repeat(visits, P)[:cfg.n_ctx]
        buckets = [(1, 2), (3, 8), (9, 32), (33, 128)]
        for name, (_, grads, _, _) in runs.items():
            errs = {}
            for which, (x, r) in (("dk", (grads[l][0], ref["dk"])), ("dv", (grads[l][1], ref["dv"]))):
                scale = np.abs(r).max()
                e = np.abs(x.astype(np.float64) - r).max(axis=(1, 2)) / scale
                errs[which] = e.max()
                by = {f"{a}-{b}": float(e[(vis_tok >= a) & (vis_tok <= b)].max(initial=0.0))
                      for a, b in buckets}
                print(f"layer {l} {name} {which}: {errs[which]:.2e}; by visits "
                      + ", ".join(f"{k}: {v:.1e}" for k, v in by.items()), flush=True)
            assert max(errs.values()) < 1e-2, (name, errs)
        g_hbm = runs["all-HBM"][1][l]
        g_f32 = runs["fp32 tier"][1][l]
        assert rel_err(g_f32[0], g_hbm[0]) < 1e-5 and rel_err(g_f32[1], g_hbm[1]) < 1e-5


def test_prefix_prefetch_ahead_of_the_append():
    """A forward sweep prefetches a layer's pages before its chunk is
    appended (prefix up to the chunk's end): the append then writes the rows
    into the window too, and the chunk's attention over the window equals the
    all-HBM pool's, bit for bit, and the oracle.  Rows past the prefix are not
    in the window: attention on them is PKV_ESTATE."""
    import torch
    import paged_kv_cache_chunk_amd as pkv
    cfg = SMALL
    f = Workload(cfg).full()
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    host = pkv.pkv_pool_create(2, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16,
                               host_tier=1)
    res = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16)
    outs = {}
    for name, pool in (("host", host), ("hbm", res)):
        pkv.pkv_append_kv(pool, 0, 0, dev(f.k[:3072]), dev(f.v[:3072]))
        if name == "host":
            pkv.pkv_prefetch_prefix(pool, 0, 4096)        # 1024 keys not appended yet
        pkv.pkv_append_kv(pool, 0, 3072, dev(f.k[3072:4096]), dev(f.v[3072:4096]))
        q = dev(f.q[3072:4096])
        o = torch.empty_like(q)
        lse = torch.empty(cfg.hq, 1024, device="cuda")
        pkv.pkv_attn_fwd(pool, 0, 3072, q, o, lse, cfg.scale)
        torch.cuda.synchronize()
        outs[name] = (o.float().cpu().numpy(), lse.cpu().numpy())
    assert np.array_equal(outs["host"][0], outs["hbm"][0])
    assert np.array_equal(outs["host"][1], outs["hbm"][1])
    O_ref, _ = oracle.attn_fwd(f.q[3072:4096], f.k, f.v, 3072, cfg.scale, cfg.page)
    assert rel_err(outs["host"][0], O_ref) < 1e-2
    pkv.pkv_append_kv(host, 0, 4096, dev(f.k[4096:4224]), dev(f.v[4096:4224]))
    q = dev(f.q[4096:4224])
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_fwd(host, 0, 4096, q, torch.empty_like(q),
                         torch.empty(cfg.hq, 128, device="cuda"), cfg.scale)
    assert e.value.status == 4, str(e.value)
    torch.cuda.synchronize()
    host.close()
    res.close()


def test_selections_made_ahead_give_the_same_sweep():
    """The backward sweep reusing selections made before it (as a forward
    sweep makes them) gives the results of selecting layer by layer inside
    it: O, LSE, dQ and the selections bit for bit, dK/dV to atomic order."""
    import paged_kv_cache_chunk_amd as pkv
    cfg = CFG.replace(n_layers=2)
    # fp32 host gradients: the two runs differ only in the order of fp32 adds
    a, ga, _, _ = _sweep(cfg, True, pkv.PKV_F32, lookahead=True, select_ahead=True)
    b, gb, _, _ = _sweep(cfg, True, pkv.PKV_F32, lookahead=True)
    for key in b:
        for name in ("O", "lse", "dq"):
            assert np.array_equal(a[key][name].numpy(), b[key][name].numpy()), (key, name)
        for x, y in zip(a[key]["sel"], b[key]["sel"]):
            assert np.array_equal(x.numpy(), y.numpy())
    for l in range(cfg.n_layers):
        assert rel_err(ga[l][0], gb[l][0]) < 1e-5 and rel_err(ga[l][1], gb[l][1]) < 1e-5
