"""GPU: argument and state checks of the C ABI return their documented
status before anything is enqueued, and a rejected call leaves the pool
usable (a following valid call still matches the oracle).  Also the
degenerate chunk n_q = 0 (a no-op)."""
import numpy as np
import pytest

import oracle
from synthetic import Workload, get_config
from tests.gpu_util import gpu_available, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _status(exc_info):
    return str(exc_info.value).split(":")[0]


def test_rejected_calls_and_recovery():
    import torch
    import paged_kv_cache_chunk_amd as pkv

    cfg = get_config("tiny_f32")  # 512 tokens, pages of 16, Hq 2 / Hkv 1, d 64, fp32
    w = Workload(cfg)
    f32 = torch.float32

    def expect(status, fn, *a, **kw):
        with pytest.raises(pkv.PkvError) as e:
            fn(*a, **kw)
        assert _status(e) == status, str(e.value)
        assert pkv.pkv_last_error()

    # pool creation
    expect("PKV_EINVAL", pkv.pkv_pool_create, 1, 1, 64, 16, 32, 16, pkv.PKV_F32)  # slots < pages
    expect("PKV_EUNSUPPORTED", pkv.pkv_pool_create, 1, 1, 96, 16, 32, 40, pkv.PKV_F32)
    expect("PKV_EUNSUPPORTED", pkv.pkv_pool_create, 1, 1, 128, 64, 8, 8, pkv.PKV_BF16)

    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_F32)
    tab = w.table()[0]
    bad = np.array(tab, dtype=np.int32).copy()
    bad[1] = bad[0]
    expect("PKV_EINVAL", pkv.pkv_page_table_set, pool, 0, 0, bad)          # slot used twice
    expect("PKV_EINVAL", pkv.pkv_page_table_set, pool, 0, 1, tab)          # no KV head 1
    pkv.pkv_page_table_set(pool, 0, 0, tab)
    chunks = [w.chunk(c) for c in range(cfg.n_chunks)]
    dev = lambda x: torch.from_numpy(x).cuda()
    ch0 = chunks[0]
    expect("PKV_ESTATE", pkv.pkv_append_kv, pool, 0, 16, dev(ch0.k), dev(ch0.v))  # not at the end
    for ch in chunks:
        pkv.pkv_append_kv(pool, 0, ch.q_pos0, dev(ch.k), dev(ch.v))
    expect("PKV_ESTATE", pkv.pkv_page_table_set, pool, 0, 0, tab)          # layer holds tokens
    big = torch.zeros(cfg.page, cfg.hkv, cfg.d, dtype=f32, device="cuda")
    expect("PKV_ECAPACITY", pkv.pkv_append_kv, pool, 0, cfg.n_ctx, big, big)  # past the table

    ch = chunks[-1]
    q, do = dev(ch.q), dev(ch.do)
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, ch.n_q, dtype=f32, device="cuda")
    dq = torch.empty_like(q)
    expect("PKV_EINVAL", pkv.pkv_attn_fwd, pool, 0, ch.q_pos0 + 1, q, o, lse, cfg.scale)  # unaligned
    expect("PKV_ESTATE", pkv.pkv_attn_fwd, pool, 0, ch.q_pos0 + cfg.page, q, o, lse, cfg.scale)
    q3 = torch.zeros(ch.n_q, 3, cfg.d, dtype=f32, device="cuda")
    pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, q3[:, :2].contiguous(), o, lse, cfg.scale)  # 2 heads fine
    with pytest.raises(ValueError):
        pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, q.transpose(0, 1), o, lse, cfg.scale)  # not contiguous
    with pytest.raises(ValueError):
        pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, q.cpu(), o, lse, cfg.scale)  # host tensor
    nqp = -(-ch.n_q // cfg.page)
    sel_bad = (torch.zeros(nqp + 1, cfg.hkv, 4, dtype=torch.int32, device="cuda"),
               torch.zeros(nqp + 1, cfg.hkv, dtype=torch.int32, device="cuda"))
    expect("PKV_EINVAL", pkv.pkv_attn_fwd, pool, 0, ch.q_pos0, q, o, lse, cfg.scale, sel=sel_bad)
    sp, sc = (torch.empty(nqp, cfg.hkv, 2, dtype=torch.int32, device="cuda"),
              torch.empty(nqp, cfg.hkv, dtype=torch.int32, device="cuda"))
    expect("PKV_EINVAL", pkv.pkv_select_topk_pages, pool, 0, ch.q_pos0, q, 4, sp, sc)  # stride 2 < 7
    expect("PKV_EINVAL", pkv.pkv_grad_zero, pool, 3)
    expect("PKV_EINVAL", pkv.pkv_read_pages, pool, 0, 9, o)

    # n_q = 0: a no-op
    e0 = torch.empty(0, cfg.hq, cfg.d, dtype=f32, device="cuda")
    pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, e0, e0, torch.empty(cfg.hq, 0, device="cuda"), cfg.scale)

    # the pool still works: one chunk's forward against the oracle
    pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, q, o, lse, cfg.scale)
    torch.cuda.synchronize()
    f = w.full()
    O_ref, _ = oracle.attn_fwd(f.q[ch.q_pos0:], f.k, f.v, ch.q_pos0, cfg.scale, cfg.page)
    assert rel_err(o.cpu().numpy(), O_ref) <= 1e-5
    pool.close()


@pytest.mark.parametrize("host_tier", [0, 1])
def test_failed_pool_creation_releases_everything(host_tier):
    """Every allocation of a pool creation, failed in turn through the
    library's test hook (PKV_FAIL_ALLOC_AT=n: the n-th device or pinned
    allocation fails as if memory were exhausted), returns PKV_ENOMEM and
    releases what the half-built pool had allocated: device free memory is
    back at its level before the attempts, and a pool created afterwards
    works (its forward matches the oracle)."""
    import os
    import torch
    import paged_kv_cache_chunk_amd as pkv

    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    kw = dict(host_tier=1, host_grad_accumulate=1, window_slots=36) if host_tier else {}
    failed = 0
    for n in range(1, 80):
        os.environ["PKV_FAIL_ALLOC_AT"] = str(n)
        try:
            pool = pkv.pkv_pool_create(2, 4, 128, 128, 64, 64, pkv.PKV_BF16, **kw)
        except pkv.PkvError as e:
            assert e.status == 2 and "injected" in str(e), str(e)
            failed += 1
            continue
        finally:
            del os.environ["PKV_FAIL_ALLOC_AT"]
        pool.close()  # n past the last allocation: created normally
        break
    assert failed >= (20 if host_tier else 6), failed
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free1 - free0) < (64 << 20), (free0, free1)
    cfg = get_config("tiny_f32")
    w = Workload(cfg)
    f = w.full()
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_F32,
                               host_tier=host_tier)
    dev = lambda x: torch.from_numpy(x).cuda()
    pkv.pkv_append_kv(pool, 0, 0, dev(f.k), dev(f.v))
    if host_tier:
        pkv.pkv_prefetch_pages(pool, 0)
    q = dev(f.q[128:256])
    o = torch.empty_like(q)
    lse = torch.empty(cfg.hq, 128, device="cuda")
    pkv.pkv_attn_fwd(pool, 0, 128, q, o, lse, cfg.scale)
    torch.cuda.synchronize()
    O_ref, _ = oracle.attn_fwd(f.q[128:256], f.k, f.v, 128, cfg.scale, cfg.page)
    assert rel_err(o.cpu().numpy(), O_ref) <= 1e-5
    pool.close()
