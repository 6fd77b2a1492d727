"""Pins of the fp64 oracle against things other than itself: brute force,
finite differences, torch's CPU scaled-dot-product attention, closed forms,
invariants and a hand-worked fixture.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.brute import attn_brute, brute_select
from synthetic import Workload, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _micro(seed=1, N=24, hq=2, hkv=1, d=8):
    r = np.random.default_rng(seed)
    return (r.standard_normal((N, hq, d)), r.standard_normal((N, hkv, d)),
            r.standard_normal((N, hkv, d)), r.standard_normal((N, hq, d)))


def _rel(a, b):
    return np.abs(np.asarray(a) - np.asarray(b)).max() / max(np.abs(np.asarray(b)).max(), 1e-300)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2)])
def test_brute_dense(hq, hkv):
    q, k, v, do = _micro(2, N=24, hq=hq, hkv=hkv)
    r = oracle.run_chunks(q, k, v, do, chunk=8, scale=0.35, page=4)
    b = attn_brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 8, 0.35, 4)
    for name, i in [("O", 0), ("lse", 1), ("dq", 2), ("dk", 3), ("dv", 4)]:
        assert np.abs(np.array(b[i]) - r[name]).max() < 1e-13, name


def test_brute_sparse():
    q, k, v, do = _micro(3, N=40, hq=4, hkv=2)
    sp = dict(top_k=2, n_sink=1, n_local=2)
    r = oracle.run_chunks(q, k, v, do, chunk=8, scale=0.35, page=4, sparse=sp)
    sels = [[[int(x) for x in s] for s in row] for row in [None] * 0] or \
        [[[list(map(int, s)) for s in row] for row in sel] for sel in r["sel"]]
    b = attn_brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 8, 0.35, 4, sels)
    for name, i in [("O", 0), ("lse", 1), ("dq", 2), ("dk", 3), ("dv", 4)]:
        assert np.abs(np.array(b[i]) - r[name]).max() < 1e-13, name
    # the selection is genuinely sparse somewhere
    assert any(len(s) < (8 * c // 4 + 2) for c, sel in enumerate(r["sel"]) for row in sel for s in row)


# ------------------------------------------------------------ selection pins
def test_select_vs_sorted():
    r = np.random.default_rng(5)
    for trial in range(6):
        page, hkv, hq, d = 4, 2, 4, 6
        N = 64
        q = r.standard_normal((N, hq, d))
        k = r.standard_normal((N, hkv, d))
        if trial % 2:  # duplicate pages -> exact ties
            for j in range(2, N // page, 3):
                k[j * page:(j + 1) * page] = k[(j - 1) * page:j * page]
        for q_pos0 in (16, 48):
            for top_k in (0, 1, 3, 100):
                a = oracle.select_pages(q[q_pos0:q_pos0 + 16], k, q_pos0, page, hkv, top_k)
                b = brute_select(q[q_pos0:q_pos0 + 16].tolist(), k.tolist(), q_pos0, page, hkv, top_k)
                assert [[list(map(int, s)) for s in row] for row in a] == b


def test_select_golden_ties():
    with open(os.path.join(GOLDEN, "select_ties.json")) as f:
        g = json.load(f)
    q = np.array(g["q"])
    k = np.array(g["k"])
    for case in g["cases"]:
        for dt in (np.float64, np.float32):
            sel = oracle.select_pages(q, k, g["q_pos0"], g["page"], g["hkv"], case["top_k"],
                                      score_dtype=dt)
            assert list(map(int, sel[0][0])) == case["expected"]


def test_select_fp32_matches_fp64_on_random():
    w = Workload(get_config("qwen_256k_topk").replace(n_ctx=4096, chunk=1024, slots=32))
    f = w.full()
    for q_pos0 in (1024, 3072):
        a, sc = oracle.select_pages(f.q[q_pos0:q_pos0 + 1024], f.k, q_pos0, 128, 4, 8,
                                    return_scores=True)
        b = oracle.select_pages(f.q[q_pos0:q_pos0 + 1024], f.k, q_pos0, 128, 4, 8,
                                score_dtype=np.float32)
        for i in range(len(a)):
            for g in range(4):
                diff = set(a[i][g].tolist()) ^ set(b[i][g].tolist())
                if diff:  # only allowed inside the 1e-5 score gap
                    cand, s = sc[(i, g)]
                    kth = np.sort(s)[::-1][min(8, len(s)) - 1]
                    for j in diff:
                        assert abs(s[list(cand).index(j)] - kth) < 1e-5


# ------------------------------------------------------ finite differences
def _loss(q, k, v, do, chunk, scale, page, sels=None):
    r = oracle.run_chunks(q, k, v, do, chunk, scale, page, sels=sels)
    return float((r["O"] * do).sum()), r


@pytest.mark.parametrize("sparse", [False, True])
def test_finite_differences_every_coordinate(sparse):
    q, k, v, do = _micro(7, N=16, hq=2, hkv=1, d=4)
    chunk, scale, page = 8, 0.4, 4
    sels = None
    if sparse:
        sels = oracle.run_chunks(q, k, v, do, chunk, scale, page,
                                 sparse=dict(top_k=1))["sel"]
    _, r = _loss(q, k, v, do, chunk, scale, page, sels)
    eps = 1e-6
    for name, x, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp, _ = _loss(q, k, v, do, chunk, scale, page, sels)
            x[idx] = old - eps
            lm, _ = _loss(q, k, v, do, chunk, scale, page, sels)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert _rel(grad, num) < 1e-7, name


def test_finite_differences_directional_tiny_config():
    cfg = get_config("tiny_f32")
    f = Workload(cfg).full()
    q, k, v, do = (x.astype(np.float64) for x in (f.q, f.k, f.v, f.do))
    _, r = _loss(q, k, v, do, cfg.chunk, cfg.scale, cfg.page)
    rng = np.random.default_rng(11)
    eps = 1e-5
    for name, x, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        u = rng.standard_normal(x.shape)
        x += eps * u
        lp, _ = _loss(q, k, v, do, cfg.chunk, cfg.scale, cfg.page)
        x -= 2 * eps * u
        lm, _ = _loss(q, k, v, do, cfg.chunk, cfg.scale, cfg.page)
        x += eps * u
        num = (lp - lm) / (2 * eps)
        ana = float((grad * u).sum())
        assert abs(num - ana) / abs(ana) < 1e-7, name


# ------------------------------------------------ independent library routine
def test_against_torch_sdpa_tiny_config():
    torch = pytest.importorskip("torch")
    cfg = get_config("tiny_f32")
    f = Workload(cfg).full()
    G = cfg.group
    q = torch.tensor(f.q, dtype=torch.float64).permute(1, 0, 2).contiguous().requires_grad_()
    k = torch.tensor(f.k, dtype=torch.float64).permute(1, 0, 2).contiguous().requires_grad_()
    v = torch.tensor(f.v, dtype=torch.float64).permute(1, 0, 2).contiguous().requires_grad_()
    do = torch.tensor(f.do, dtype=torch.float64).permute(1, 0, 2)
    kr = k.repeat_interleave(G, dim=0)
    vr = v.repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], kr[None], vr[None], is_causal=True, scale=cfg.scale)[0]
    (o * do).sum().backward()
    r = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page)
    assert _rel(r["O"], o.detach().permute(1, 0, 2).numpy()) < 1e-12
    assert _rel(r["dq"], q.grad.permute(1, 0, 2).numpy()) < 1e-12
    assert _rel(r["dk"], k.grad.permute(1, 0, 2).numpy()) < 1e-12
    assert _rel(r["dv"], v.grad.permute(1, 0, 2).numpy()) < 1e-12


# ---------------------------------------------------------------- invariants
def test_chunked_equals_full_sequence():
    cfg = get_config("tiny_f32")
    f = Workload(cfg).full()
    a = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.chunk, cfg.scale, cfg.page)
    b = oracle.run_chunks(f.q, f.k, f.v, f.do, cfg.n_ctx, cfg.scale, cfg.page)
    for name in ("O", "lse", "dq", "dk", "dv"):
        assert _rel(a[name], b[name]) < 1e-12, name


def test_page_table_permutation_invariance():
    cfg = get_config("tiny_f32")
    w = Workload(cfg)
    f = w.full()
    ident = np.arange(cfg.n_pages, dtype=np.int32)[None, :]
    outs = []
    for table in (ident, w.table()):
        kp = oracle.page_in(f.k, table, cfg.slots, cfg.page)
        vp = oracle.page_in(f.v, table, cfg.slots, cfg.page)
        k = oracle.depage(kp, table, cfg.n_ctx)
        v = oracle.depage(vp, table, cfg.n_ctx)
        outs.append(oracle.run_chunks(f.q, k, v, f.do, cfg.chunk, cfg.scale, cfg.page))
    assert not np.array_equal(ident[0], w.table()[0])
    for name in ("O", "lse", "dq", "dk", "dv"):
        assert np.array_equal(outs[0][name], outs[1][name]), name


def test_topk_all_pages_equals_dense():
    q, k, v, do = _micro(9, N=48, hq=4, hkv=2, d=8)
    a = oracle.run_chunks(q, k, v, do, 16, 0.3, 4)
    b = oracle.run_chunks(q, k, v, do, 16, 0.3, 4, sparse=dict(top_k=12))
    for name in ("O", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("sparse", [None, dict(top_k=2)])
def test_gradient_sum_identities(sparse):
    q, k, v, do = _micro(13, N=64, hq=4, hkv=2, d=8)
    r = oracle.run_chunks(q, k, v, do, 16, 0.3, 4, sparse=sparse)
    G = 2
    for g in range(2):
        assert np.abs(r["dk"][:, g].sum(0)).max() < 1e-12 * np.abs(r["dk"]).max() * 64
        want = do[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        assert _rel(r["dv"][:, g].sum(0), want) < 1e-12


def test_closed_forms():
    q, k, v, do = _micro(17, N=32, hq=2, hkv=1, d=8)
    scale = 0.3
    r = oracle.run_chunks(q, k, v, do, 8, scale, 4)
    # first row sees only key 0
    for h in range(2):
        assert np.allclose(r["O"][0, h], v[0, 0], atol=1e-15)
        assert abs(r["lse"][h, 0] - scale * q[0, h] @ k[0, 0]) < 1e-14
    # zero keys -> uniform attention over s <= t
    z = oracle.run_chunks(q, np.zeros_like(k), v, do, 8, scale, 4)
    cm = np.cumsum(v[:, 0], axis=0) / np.arange(1, 33)[:, None]
    for h in range(2):
        assert np.abs(z["O"][:, h] - cm).max() < 1e-14
        assert np.abs(z["lse"][h] - np.log(np.arange(1, 33))).max() < 1e-14


def test_hand_worked_two_tokens():
    """d=2, tau=1/sqrt(2).  k0=0, k1=(1,0), q1=(sqrt2*ln3, 0) so row 1 has
    logits (0, ln3) and P=(1/4, 3/4); v0=(1,0), v1=(0,1); dO1=(1,0), dO0=0.
    By hand: O1=(1/4,3/4), LSE1=ln4, O0=v0, LSE0=0; D=1/4; dS1=(3/16,-3/16);
    dQ1=-3/(16 sqrt2) k1; dK0=(3 ln3/16, 0), dK1=-dK0; dV0=(1/4,0), dV1=(3/4,0)."""
    s2 = math.sqrt(2.0)
    q = np.array([[[1.0, 0.0]], [[s2 * math.log(3.0), 0.0]]])
    k = np.array([[[0.0, 0.0]], [[1.0, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    do = np.array([[[0.0, 0.0]], [[1.0, 0.0]]])
    for chunk in (1, 2):
        r = oracle.run_chunks(q, k, v, do, chunk, 1 / s2, 1)
        assert np.allclose(r["O"][:, 0], [[1, 0], [0.25, 0.75]], atol=1e-15)
        assert np.allclose(r["lse"][0], [0.0, math.log(4.0)], atol=1e-15)
        assert np.allclose(r["dq"][:, 0], [[0, 0], [-3 / (16 * s2), 0]], atol=1e-15)
        l3 = 3 * math.log(3.0) / 16
        assert np.allclose(r["dk"][:, 0], [[l3, 0], [-l3, 0]], atol=1e-15)
        assert np.allclose(r["dv"][:, 0], [[0.25, 0], [0.75, 0]], atol=1e-15)


# ------------------------------------------------------- sampled helpers
@pytest.mark.parametrize("sparse", [None, dict(top_k=2)])
def test_sampled_helpers_match_full(sparse):
    q, k, v, do = _micro(21, N=64, hq=4, hkv=2, d=8)
    chunk, page, scale = 16, 4, 0.3
    r = oracle.run_chunks(q, k, v, do, chunk, scale, page, sparse=sparse)
    rows = np.array([0, 5, 17, 40, 63])
    for h in range(4):
        ok = None
        if sparse:
            ok = np.zeros((len(rows), 16), dtype=bool)
            for n, t in enumerate(rows):
                ok[n, r["sel"][t // chunk][(t % chunk) // page][h // 2]] = True
        O, lse, dq = oracle.rows_fwd_bwd(q[rows, h], do[rows, h], rows, h, k, v, scale, 2,
                                         page, ok)
        assert _rel(O, r["O"][rows, h]) < 1e-13
        assert np.abs(lse - r["lse"][h, rows]).max() < 1e-13
        assert _rel(dq, r["dq"][rows, h]) < 1e-13
    s0 = 40
    dk, dv = oracle.key_grads_sampled(s0, q[s0:], do[s0:], k, v, scale, chunk, page,
                                      r["sel"])
    assert _rel(dk, r["dk"][s0:]) < 1e-13
    assert _rel(dv, r["dv"][s0:]) < 1e-13


def test_chunk_page_grads_against_brute_force_and_masked_form():
    """One top-K chunk's contribution to chosen key pages (keys gathered per
    selection) equals the per-(t, h, s) loops of the brute-force oracle run on
    that chunk alone, and the masked full-key form."""
    q, k, v, do = _micro(23, N=48, hq=4, hkv=2, d=8)
    chunk, page, scale = 16, 4, 0.3
    sp = dict(top_k=2, n_sink=1, n_local=2)
    r = oracle.run_chunks(q, k, v, do, chunk, scale, page, sparse=sp)
    c = 2                              # last chunk: rows 32..47, keys 0..47
    q_pos0 = c * chunk
    sel = r["sel"][c]
    pages = [0, 3, 5, 11]             # sink, earlier pages, the last query page
    dk, dv = oracle.chunk_page_grads(q[q_pos0:], do[q_pos0:], q_pos0, k, v, scale, page, sel,
                                     pages)
    n = q_pos0 + chunk
    # brute force (per-(t, h, s) loops) over the chunks up to this one, with
    # dO = 0 on the rows of earlier chunks: they then add nothing to dK/dV,
    # which leaves this chunk's contribution
    doz = np.zeros_like(do[:n])
    doz[q_pos0:] = do[q_pos0:n]
    sels_b = [[[list(map(int, s_)) for s_ in row] for row in r["sel"][cc]] for cc in range(c + 1)]
    b = attn_brute(q[:n].tolist(), k[:n].tolist(), v[:n].tolist(), doz.tolist(), chunk, scale,
                   page, sels_b)
    bk, bv = np.array(b[3]), np.array(b[4])
    for j, p_ in enumerate(pages):
        sl = slice(p_ * page, (p_ + 1) * page)
        assert np.abs(dk[j] - bk[sl]).max() < 1e-13 and np.abs(dv[j] - bv[sl]).max() < 1e-13
    # the masked form of one chunk (attn_bwd over all keys up to the chunk)
    m = oracle.attn_bwd(q[q_pos0:n], k, v, do[q_pos0:n], q_pos0, scale, page, sel)
    for j, p_ in enumerate(pages):
        sl = slice(p_ * page, (p_ + 1) * page)
        assert _rel(dk[j], m["dk"][sl]) < 1e-13 and _rel(dv[j], m["dv"][sl]) < 1e-13
    # the sink page is held by every query page, so it did receive gradient
    assert np.abs(dv[0]).max() > 0


def test_page_in_depage_roundtrip_and_pool_bytes():
    cfg = get_config("tiny_f32")
    w = Workload(cfg)
    f = w.full()
    pool = oracle.page_in(f.k, w.table(), cfg.slots, cfg.page)
    assert pool.shape == (1, 40, 16, 64)
    assert np.array_equal(oracle.depage(pool, w.table(), cfg.n_ctx), f.k)
    # the 1M-token offloaded workload: 28 layers x 2^20 tokens x 4 KV heads x
    # 128 x (K+V) bf16 plus the same again for bf16 gradients ~= 115 GB
    c4 = get_config("qwen_1m_offload")
    kv = c4.n_layers * c4.n_ctx * c4.hkv * c4.d * 2 * 2
    assert kv == 56 * 2 ** 30
    assert abs(2 * kv / 1e9 - 120.3) < 0.1
