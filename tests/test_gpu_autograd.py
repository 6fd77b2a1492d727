"""GPU: the autograd wrapper (paged_kv_cache_chunk_amd.autograd) gives the
same o and q.grad (bit for bit) and pool dK/dV (up to the order of fp32
atomic adds) as direct pkv_attn_fwd / pkv_attn_bwd calls,
and a whole chunk-recurrent run through it matches the oracle."""
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


def _pool(cfg, w, dt):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    kvd = pkv.PKV_BF16 if cfg.dtype == "bf16" else pkv.PKV_F32
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, kvd)
    tab = w.table()
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    chunks = [w.chunk(c) for c in range(cfg.n_chunks)]
    for ch in chunks:
        pkv.pkv_append_kv(pool, 0, ch.q_pos0, torch.from_numpy(ch.k).to(dt).cuda(),
                          torch.from_numpy(ch.v).to(dt).cuda())
    return pool, chunks


def _grads(pool, cfg):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dv)
    torch.cuda.synchronize()
    return dk.cpu().numpy(), dv.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_f32", "qwen_mini_bf16"])
def test_autograd_matches_direct_calls(name):
    import torch
    import paged_kv_cache_chunk_amd as pkv
    from paged_kv_cache_chunk_amd.autograd import paged_attention

    cfg = get_config("tiny_f32") if name == "tiny_f32" else \
        mini_config("qwen_32k_dense", n_ctx=640, chunk=256)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = Workload(cfg)
    pool, chunks = _pool(cfg, w, dt)
    ch = chunks[-1]
    q = torch.from_numpy(ch.q).to(dt).cuda()
    do = torch.from_numpy(ch.do).to(dt).cuda()

    # direct calls
    o_ref = torch.empty_like(q)
    lse = torch.empty(cfg.hq, ch.n_q, dtype=torch.float32, device="cuda")
    dq_ref = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    pkv.pkv_attn_fwd(pool, 0, ch.q_pos0, q, o_ref, lse, cfg.scale)
    pkv.pkv_attn_bwd(pool, 0, ch.q_pos0, q, o_ref, do, lse, dq_ref, cfg.scale)
    torch.cuda.synchronize()
    dk_ref, dv_ref = _grads(pool, cfg)

    # the same through autograd, on a zeroed gradient pool
    pkv.pkv_grad_zero(pool, 0)
    qa = q.clone().requires_grad_(True)
    o = paged_attention(qa, pool, 0, ch.q_pos0, cfg.scale)
    (o.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    dk, dv = _grads(pool, cfg)
    assert torch.equal(o, o_ref)
    assert qa.grad.dtype == q.dtype
    assert torch.equal(qa.grad, dq_ref.to(dt))
    # dK/dV: the same contributions; fp32 atomics of split workgroups may add
    # them in another order
    assert rel_err(dk, dk_ref) <= 1e-5 and rel_err(dv, dv_ref) <= 1e-5
    pool.close()


def test_autograd_chunk_recurrent_run_matches_oracle():
    """Every chunk through the autograd wrapper, last to first: O, q.grad and
    the pool's dK/dV against the fp64 oracle of the whole sequence."""
    import torch
    from paged_kv_cache_chunk_amd.autograd import paged_attention

    cfg = get_config("tiny_f32")
    w = Workload(cfg)
    pool, chunks = _pool(cfg, w, torch.float32)
    N = cfg.n_ctx
    O = np.zeros((N, cfg.hq, cfg.d))
    dq = np.zeros((N, cfg.hq, cfg.d))
    for ch in reversed(chunks):
        q = torch.from_numpy(ch.q).cuda().requires_grad_(True)
        do = torch.from_numpy(ch.do).cuda()
        o = paged_attention(q, pool, 0, ch.q_pos0, cfg.scale)
        (o * do).sum().backward()
        sl = slice(ch.q_pos0, ch.q_pos0 + ch.n_q)
        O[sl] = o.detach().cpu().numpy()
        dq[sl] = q.grad.cpu().numpy()
    dk, dv = _grads(pool, cfg)
    f = w.full()
    ref = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page)
    for got, name in ((O, "O"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert rel_err(got, ref[name]) <= 1e-5, name
    pool.close()
