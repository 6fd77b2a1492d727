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


def _reference(block, x, gy):
    x = x.detach().float().clone().requires_grad_()
    wq, wk, wv, wo = [w.detach().clone().requires_grad_() for w in block.parameters()]
    N, hq, hkv, d = x.shape[0], block.hq, block.hkv, block.d
    f32 = lambda t: t.float()
    q = block._rope((x @ wq.t()).view(N, hq, d), 0).float()
    k = block._rope((x @ wk.t()).view(N, hkv, d), 0).float()
    v = (x @ wv.t()).view(N, hkv, d)
    causal = torch.ones(N, N, dtype=torch.bool, device=x.device).tril()
    outs = []
    for h in range(hq):
        g = h // (hq // hkv)
        s = (q[:, h] @ k[:, g].t().contiguous()) * block.scale
        s = s.masked_fill(~causal, float("-inf"))
        outs.append(torch.softmax(s, dim=-1) @ f32(v[:, g]))
    o = torch.stack(outs, dim=1)
    y = x + o.reshape(N, hq * d) @ wo.t()
    (y * gy.float()).sum().backward()
    return y.detach(), x.grad, [wq.grad, wk.grad, wv.grad, wo.grad]


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


def test_recurrent_block_top_k_runs():
    """Top-K mode of the same block: the sweep runs and every gradient is
    finite (the restricted attention's values are pinned by the parity
    tests)."""
    from paged_kv_cache_chunk_amd.chunks import Sparse
    from paged_kv_cache_chunk_amd.recurrent import AttentionBlock

    block = AttentionBlock(hidden=256, hq=4, hkv=2, d=128, page=128, max_tokens=2048,
                           sparse=Sparse(top_k=4), seed=2)
    x = torch.randn(2048, 256, device="cuda").to(torch.bfloat16)
    xs = [x[i:i + 512] for i in range(0, 2048, 512)]
    gys = [torch.randn_like(t) / 16 for t in xs]
    block.forward_sweep(xs)
    dxs = block.backward_sweep(xs, gys)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in dxs)
    assert all(torch.isfinite(w.grad).all() and w.grad.abs().sum() > 0 for w in block.parameters())
    block.close()
