"""GPU: the error of page top-K attention against dense attention, as a
function of the budget K, measured against the fp64 oracle ("Out of the
Memory Barrier", gist.science de, section 4: the gradient approximation error
stays acceptable at adequate retrieval budgets; sciencestack.ai, Figure 5:
on real text each query page retrieves a few key pages).

Two input laws at one KV head's share of the Qwen2.5-7B shape (7 query heads,
1 KV head, d 128), 16384 tokens in chunks of 4096, pages of 128:
  * i.i.d.: the 256K top-K workload's law (keys N(0,1) plus offsets of norm 2
    on 5% of the pages, queries N(0,1)): dense attention spreads over every
    earlier key, so no budget short of all pages approximates it;
  * structured: offsets of norm 8 on 10% of the pages, and each query page's
    queries drawn toward 4 of them (affinity 1.0): attention concentrates on a
    few pages per query page, as Figure 5 shows for real text.
For each budget the library's sparse fwd+bwd is compared with the oracle's
dense result (the approximation error: relative Frobenius norm of the
difference, and cosine similarity), and with the oracle's sparse result on
the library's own selection (the implementation error, max-abs / max |ref|,
bound 1e-2).  This test checks one budget on the structured law;
tests/budget_sweep.py runs every budget of both laws and prints the table."""
import numpy as np
import pytest

import oracle
from synthetic import Workload, mini_config
from tests.gpu_util import compare_selection, gpu_available, rel_err, run_layer, sel_lists

pytestmark = pytest.mark.gpu

BASE = dict(n_ctx=16384, chunk=4096, hq=7, hkv=1)
LAWS = {
    "iid": mini_config("qwen_256k_topk", **BASE),
    "structured": mini_config("qwen_256k_topk", **BASE, planted_norm=8.0, planted_frac=0.1,
                              query_targets=4, query_affinity=1.0),
}
NAMES = ("O", "dq", "dk", "dv")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _fro(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def _cos(x, ref):
    x, ref = np.asarray(x, np.float64).ravel(), np.asarray(ref, np.float64).ravel()
    return float(x @ ref / (np.linalg.norm(x) * np.linalg.norm(ref)))


def _budget(cfg, f, dense, top_k):
    """Library sparse run at budget top_k; its errors against the oracle's
    dense result and against the oracle's sparse result on its selection."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    w = Workload(cfg.replace(top_k=top_k))
    got = run_layer(w.cfg, w, sparse=Sparse(top_k=top_k))
    got["pool"].close()
    sels = []
    for c in range(cfg.n_chunks):
        q_pos0, n = cfg.chunk_range(c)
        ref_sel, scores = oracle.select_pages(f.q[q_pos0:q_pos0 + n], f.k, q_pos0, cfg.page,
                                              cfg.hkv, top_k, cfg.n_sink, cfg.n_local,
                                              score_dtype=np.float32, return_scores=True)
        gsel = sel_lists(got["sel"][c])
        compare_selection(gsel, ref_sel, scores, top_k)  # 1e-5 gap rule, asserted inside
        sels.append([[np.array(x, dtype=np.int64) for x in row] for row in gsel])
    sparse = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page, sels=sels)
    pairs = sum(len(x) for s in sels for row in s for x in row)
    dense_pages = sum(i + 1 for i in range(cfg.n_pages))
    return {
        "impl": {n: rel_err(got[n], sparse[n]) for n in NAMES},
        "approx": {n: _fro(got[n], dense[n]) for n in NAMES},
        "approx_oracle": {n: _fro(sparse[n], dense[n]) for n in NAMES},
        "cos": {n: _cos(got[n], dense[n]) for n in NAMES},
        "page_frac": pairs / (dense_pages * cfg.hkv),
    }


def _dense(cfg):
    f = Workload(cfg).full()
    return f, oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page)


def test_structured_budget_error():
    """Structured law, K = 16: implementation error within 1e-2 of the
    oracle on the library's selection, and the top-K result within 5% (relative
    Frobenius norm) of dense attention for O, dQ, dK and dV."""
    cfg = LAWS["structured"]
    f, dense = _dense(cfg)
    r = _budget(cfg, f, dense, 16)
    print({k: ({n: f"{v:.2e}" for n, v in d.items()} if isinstance(d, dict) else d)
           for k, d in r.items()}, flush=True)
    for n in NAMES:
        assert r["impl"][n] <= 1e-2, (n, r["impl"][n])
        assert r["approx"][n] <= 0.05, (n, r["approx"][n])
