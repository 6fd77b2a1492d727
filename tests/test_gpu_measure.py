"""GPU: the measurement kernels run through the C ABI and touch what they
document (pkv_measure_atomics adds `value` reps times to exactly the keys
below n_keys; pkv_measure_gather reads without writing the pool)."""
import numpy as np
import pytest

from synthetic import Workload, mini_config
from tests.gpu_util import gpu_available

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def test_measure_kernels():
    import torch
    import paged_kv_cache_chunk_amd as pkv

    cfg = mini_config("qwen_32k_dense", n_ctx=640, chunk=256)
    w = Workload(cfg)
    pool = pkv.pkv_pool_create(1, cfg.hkv, cfg.d, cfg.page, cfg.n_pages, cfg.slots, pkv.PKV_BF16)
    tab = w.table()
    for g in range(cfg.hkv):
        pkv.pkv_page_table_set(pool, 0, g, tab[g])
    for c in range(cfg.n_chunks):
        ch = w.chunk(c)
        pkv.pkv_append_kv(pool, 0, ch.q_pos0, torch.from_numpy(ch.k).to(torch.bfloat16).cuda(),
                          torch.from_numpy(ch.v).to(torch.bfloat16).cuda())
    k_before = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_read_pages(pool, 0, pkv.PKV_K, k_before)
    q_pos0, n_q = cfg.chunk_range(cfg.n_chunks - 1)
    out = torch.zeros(-(-n_q // 128) * cfg.hq, dtype=torch.float32, device="cuda")
    pkv.pkv_measure_gather(pool, 0, q_pos0, n_q, cfg.hq, out)
    n_keys = 300  # a partial slab and a partial page
    pkv.pkv_measure_atomics(pool, 0, n_keys, 3, 1.0)
    dk = torch.empty(cfg.n_ctx, cfg.hkv, cfg.d, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    k_after = torch.empty_like(k_before)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DK, dk)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_DV, dv)
    pkv.pkv_read_pages(pool, 0, pkv.PKV_K, k_after)
    torch.cuda.synchronize()
    dk, dv = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.all(dk[:n_keys] == 3.0) and np.all(dv[:n_keys] == 3.0)
    assert np.all(dk[n_keys:] == 0.0) and np.all(dv[n_keys:] == 0.0)
    assert torch.equal(k_before, k_after)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_measure_atomics(pool, 0, cfg.n_ctx + 1, 1)
    pool.close()
