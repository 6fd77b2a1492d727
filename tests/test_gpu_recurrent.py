"""GPU: chunk-recurrent training of an attention block (paged_kv_cache_chunk_amd
.recurrent) gives the gradients of ordinary full-sequence training.

The reference is the same block evaluated on the whole sequence at once with
plain torch ops in fp32 (explicit causal softmax attention with grouped
query heads), differentiated by autograd: dL/dx of every token and the four
weight gradients must match the recurrent sweep, in which attention and the
KV gradients go through libpkv and the cache never enters autograd."""
import pytest
import torch

from tests.gpu_util import gpu_available

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _allowed(block, N, sels):
    """[hkv][N][N] bool: key s allowed for query t (causal; with a top-K
    selection of each chunk, also s's page listed for t's query page)."""
    causal = torch.ones(N, N, dtype=torch.bool, device="cuda").tril()
    if not sels:
        return causal[None].expand(block.hkv, N, N)
    P = block.page
    pages_ok = torch.zeros(block.hkv, N, -(-N // P), dtype=torch.bool, device="cuda")
    for pos0, (pages, count) in sels.items():
        pages, count = pages.cpu(), count.cpu()
        for il in range(pages.shape[0]):
            t0, t1 = pos0 + il * P, min(pos0 + (il + 1) * P, N)
            for g in range(block.hkv):
                pages_ok[g, t0:t1, pages[il, g, :count[il, g]].long()] = True
    key_page = torch.arange(N, device="cuda") // P
    return causal[None] & pages_ok[:, :, key_page]


def _reference(blocks, x, gy, sels=None):
    """The blocks applied one after the other to the whole sequence with
    plain torch ops in fp32 (explicit softmax attention, grouped query heads,
    the given selections held fixed), differentiated by autograd."""
    if not isinstance(blocks, (list, tuple)):
        blocks = [blocks]
    x = x.detach().float().clone().requires_grad_()
    ws = [[w.detach().clone().requires_grad_() for w in b.parameters()] for b in blocks]
    h = x
    N = x.shape[0]
    for l, b in enumerate(blocks):
        wq, wk, wv, wo = ws[l]
        hq, hkv, d = b.hq, b.hkv, b.d
        q = b._rope((h @ wq.t()).view(N, hq, d), 0).float()
        k = b._rope((h @ wk.t()).view(N, hkv, d), 0).float()
        v = (h @ wv.t()).view(N, hkv, d).float()
        ok = _allowed(b, N, (sels or [None] * len(blocks))[l])
        outs = []
        for hh in range(hq):
            g = hh // (hq // hkv)
            sc = (q[:, hh] @ k[:, g].t().contiguous()) * b.scale
            sc = sc.masked_fill(~ok[g], float("-inf"))
            outs.append(torch.softmax(sc, dim=-1) @ v[:, g])
        o = torch.stack(outs, dim=1)
        h = h + o.reshape(N, hq * d) @ wo.t()
    (h * gy.float()).sum().backward()
    dws = [[w.grad for w in wl] for wl in ws]
    return h.detach(), x.grad, (dws[0] if len(blocks) == 1 else dws)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, 2e-4), (torch.bfloat16, 3e-2)])
def test_recurrent_block_matches_full_sequence(dtype, tol):
    from paged_kv_cache_chunk_amd.recurrent import AttentionBlock

    torch.manual_seed(0)
    hidden, n_ctx, chunk = 256, 1152, 384          # 3 chunks of 384 = 3 pages each
    block = AttentionBlock(hidden=hidden, hq=4, hkv=2, d=128, page=128, max_tokens=n_ctx,
                           dtype=dtype, seed=1)
    x = torch.randn(n_ctx, hidden, device="cuda")
    gy = torch.randn(n_ctx, hidden, device="cuda") / 16
    xs = [x[i:i + chunk].to(dtype) for i in range(0, n_ctx, chunk)]
    gys = [gy[i:i + chunk].to(dtype) for i in range(0, n_ctx, chunk)]
    ys = block.forward_sweep(xs)
    dxs = block.backward_sweep(xs, gys)
    torch.cuda.synchronize()
    y_ref, dx_ref, dw_ref = _reference(block, torch.cat(xs), torch.cat(gys))

    def rel(a, b):
        return float((a.float() - b.float()).abs().max() / b.float().abs().max())
    errs = {"y": rel(torch.cat(ys), y_ref), "dx": rel(torch.cat(dxs), dx_ref)}
    for name, w, ref in zip(("dWq", "dWk", "dWv", "dWo"), block.parameters(), dw_ref):
        errs[name] = rel(w.grad, ref)
    print(dtype, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= tol, f"{name}: {e:.3e} > {tol}"
    block.close()


def test_recurrent_block_top_k_matches_reference():
    """Top-K mode of the same block: against the fp32 torch reference on the
    whole sequence with the block's own selections held fixed (the selection
    is a constant of the gradient; the parity tests pin the selection itself
    to the oracle)."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from paged_kv_cache_chunk_amd.recurrent import AttentionBlock

    torch.manual_seed(1)
    block = AttentionBlock(hidden=256, hq=4, hkv=2, d=128, page=128, max_tokens=2048,
                           sparse=Sparse(top_k=4), seed=2)
    x = torch.randn(2048, 256, device="cuda").to(torch.bfloat16)
    gy = (torch.randn(2048, 256, device="cuda") / 16).to(torch.bfloat16)
    xs = [x[i:i + 512] for i in range(0, 2048, 512)]
    gys = [gy[i:i + 512] for i in range(0, 2048, 512)]
    ys = block.forward_sweep(xs)
    dxs = block.backward_sweep(xs, gys)
    torch.cuda.synchronize()
    y_ref, dx_ref, dw_ref = _reference(block, x, gy, sels=[block.sels])

    def rel(a, b):
        return float((a.float() - b.float()).abs().max() / b.float().abs().max())
    errs = {"y": rel(torch.cat(ys), y_ref), "dx": rel(torch.cat(dxs), dx_ref)}
    for name, w, ref in zip(("dWq", "dWk", "dWv", "dWo"), block.parameters(), dw_ref):
        errs[name] = rel(w.grad, ref)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= 3e-2, f"{name}: {e:.3e}"
    block.close()


def _stack_run(dtype, sparse, host_tier, n_ctx=1536, chunk=512, layers=2, host_adds=False):
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from paged_kv_cache_chunk_amd.recurrent import AttentionStack
    torch.manual_seed(3)
    st = AttentionStack(layers, hidden=256, hq=4, hkv=2, d=128, page=128, max_tokens=n_ctx,
                        sparse=Sparse(top_k=3) if sparse else None, dtype=dtype, seed=5,
                        host_tier=host_tier, host_grad_accumulate=host_adds)
    x = torch.randn(n_ctx, 256, device="cuda")
    gy = torch.randn(n_ctx, 256, device="cuda") / 16
    xs = [x[i:i + chunk].to(dtype) for i in range(0, n_ctx, chunk)]
    gys = [gy[i:i + chunk].to(dtype) for i in range(0, n_ctx, chunk)]
    ys = st.forward_sweep(xs)
    dxs = st.backward_sweep(xs, gys)
    torch.cuda.synchronize()
    out = dict(y=torch.cat(ys).float(), dx=torch.cat(dxs).float(),
               dw=[w.grad.clone() for w in st.parameters()], st=st,
               x=torch.cat(xs), gy=torch.cat(gys))
    return out


@pytest.mark.parametrize("host_adds", [False, True])
@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_stack_host_tier_matches_resident(sparse, dtype, host_adds):
    """A two-layer stack with every layer's K/V and KV gradients in the host
    tier (fp32 host gradients; two HBM windows filled one layer ahead on a
    side stream; in dense mode the forward sweep fetches a layer before its
    chunk is appended) gives the outputs of the all-HBM stack bit for bit and
    its gradients up to the order of the fp32 additions.  host_adds: the
    backward fetches K/V only and the library's host threads add each visit's
    gradient contributions into the tier; the chunk's own dK/dV rows, which
    go back through W_k and W_v, are then the window's contributions plus the
    tier's sums."""
    off = _stack_run(dtype, sparse, True, host_adds=host_adds)
    res = _stack_run(dtype, sparse, False)
    assert torch.equal(off["y"], res["y"])

    def rel(a, b):
        return float((a.float() - b.float()).abs().max() / b.float().abs().max())
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    errs = {"dx": rel(off["dx"], res["dx"])}
    for i, (a, b) in enumerate(zip(off["dw"], res["dw"])):
        errs[f"dw{i}"] = rel(a, b)
    print(dtype, sparse, host_adds, {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= tol, (k, e)
    off["st"].close()
    res["st"].close()


@pytest.mark.parametrize("sparse", [False, True])
def test_stack_matches_full_sequence_reference(sparse):
    """The two-layer stack (fp32, host tier) against the fp32 torch reference
    of the whole sequence (top-K: each layer's selections held fixed)."""
    got = _stack_run(torch.float32, sparse, True)
    st = got["st"]
    sels = [b.sels for b in st.blocks] if sparse else None
    y_ref, dx_ref, dws = _reference(st.blocks, got["x"], got["gy"], sels=sels)

    def rel(a, b):
        return float((a.float() - b.float()).abs().max() / b.float().abs().max())
    errs = {"y": rel(got["y"], y_ref), "dx": rel(got["dx"], dx_ref)}
    flat_ref = [w for wl in dws for w in wl]
    for i, (a, b) in enumerate(zip(got["dw"], flat_ref)):
        errs[f"dw{i}"] = rel(a, b)
    print(sparse, {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= 2e-4, (k, e)
    st.close()
