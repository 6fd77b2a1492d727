"""Python binding of libpkv (paged-KV chunk attention on MI355X).

Argument marshalling only: each function below has the name of the C entry
point it calls (see include/pkv.h for the full contract), turns torch tensors
into raw device pointers and the current torch stream into a hipStream_t, and
raises PkvError when the library returns a non-OK status.  All computation
happens in libpkv's HIP kernels; if libpkv.so is missing this module raises on
first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16 = 0, 1
PKV_K, PKV_V, PKV_DK, PKV_DV, PKV_REPS = 0, 1, 2, 3, 4
STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_ENOMEM", 3: "PKV_ECAPACITY",
          4: "PKV_ESTATE", 5: "PKV_EHIP", 6: "PKV_EUNSUPPORTED"}

EXPORTS = (
    "pkv_pool_create", "pkv_pool_destroy", "pkv_page_table_set", "pkv_length",
    "pkv_append_kv", "pkv_attn_fwd", "pkv_attn_bwd", "pkv_select_topk_pages",
    "pkv_prefetch_pages", "pkv_writeback_grads", "pkv_grad_zero", "pkv_read_pages",
    "pkv_pool_bytes", "pkv_last_error", "pkv_pool_reset", "pkv_kernel_timing",
    "pkv_kernel_times", "pkv_offload_bytes", "pkv_measure_gather", "pkv_measure_atomics",
    "pkv_read_rows", "pkv_prefetch_prefix", "pkv_attn_bwd_noalloc",
)
KERNEL_KINDS = ("append", "select", "fwd", "delta", "dq", "dkdv", "fetch", "writeback")


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class pkv_pool_desc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_logical_pages", ctypes.c_int32), ("n_slots", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("host_tier", ctypes.c_int32),
        ("host_grad_dtype", ctypes.c_int32), ("host_grad_accumulate", ctypes.c_int32),
        ("window_slots", ctypes.c_int32), ("device_budget_bytes", ctypes.c_int64),
    ]


class pkv_sel(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("n_qpages", ctypes.c_int32), ("stride", ctypes.c_int32)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libpkv.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m paged_kv_cache_chunk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, VP = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_void_p)
        sig = {
            "pkv_pool_create": [ctypes.POINTER(pkv_pool_desc), ctypes.POINTER(P)],
            "pkv_pool_destroy": [P],
            "pkv_page_table_set": [P, I32, I32, VP, I32],
            "pkv_append_kv": [P, I32, I64, I64, VP, VP, VP],
            "pkv_attn_fwd": [P, I32, I64, I64, I32, F, VP, ctypes.POINTER(pkv_sel), VP, VP, VP],
            "pkv_attn_bwd": [P, I32, I64, I64, I32, F, VP, VP, VP, VP,
                             ctypes.POINTER(pkv_sel), VP, VP],
            "pkv_attn_bwd_noalloc": [P, I32, I64, I64, I32, F, VP, VP, VP, VP,
                                     ctypes.POINTER(pkv_sel), VP, VP],
            "pkv_select_topk_pages": [P, I32, I64, I64, I32, VP, I32, I32, I32, VP, VP, I32, VP],
            "pkv_prefetch_pages": [P, I32, ctypes.POINTER(pkv_sel), I32, VP, VP],
            "pkv_prefetch_prefix": [P, I32, I64, I32, VP, VP],
            "pkv_writeback_grads": [P, I32, VP, VP],
            "pkv_grad_zero": [P, I32, VP],
            "pkv_read_pages": [P, I32, I32, VP, VP],
            "pkv_pool_bytes": [P, ctypes.POINTER(I64), ctypes.POINTER(I64)],
            "pkv_measure_gather": [P, I32, I64, I64, I32, ctypes.POINTER(pkv_sel), VP, VP],
            "pkv_read_rows": [P, I32, I32, I64, I64, VP, VP],
            "pkv_measure_atomics": [P, I32, I64, I32, F, VP],
            "pkv_pool_reset": [P, I32],
            "pkv_offload_bytes": [P, ctypes.POINTER(I64), ctypes.POINTER(I64)],
            "pkv_kernel_timing": [I32],
            "pkv_kernel_times": [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.pkv_length.argtypes = [P, I32]
        L.pkv_length.restype = I64
        L.pkv_last_error.argtypes = []
        L.pkv_last_error.restype = ctypes.c_char_p
        _lib_handle = L
    return _lib_handle


def _check(status: int) -> None:
    if status != 0:
        msg = lib().pkv_last_error()
        raise PkvError(status, msg.decode() if msg else "")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpkv takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libpkv takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _sel(sel) -> Optional[pkv_sel]:
    """sel: None (dense) or (pages int32 tensor [nqp][hkv][stride], count int32 [nqp][hkv])."""
    if sel is None:
        return None
    pages, count = sel
    return pkv_sel(_ptr(pages), _ptr(count), pages.shape[0], pages.shape[2])


def _selp(sel):
    s = _sel(sel)
    return None if s is None else ctypes.byref(s)


class Pool:
    """Owning handle of a pkv_pool (destroyed on close / garbage collection)."""

    def __init__(self, handle: int, desc: pkv_pool_desc):
        self.handle = handle
        self.desc = desc

    def close(self) -> None:
        if self.handle:
            _check(lib().pkv_pool_destroy(self.handle))
            self.handle = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def pkv_pool_create(n_layers: int, n_kv_heads: int, head_dim: int, page_size: int,
                    max_logical_pages: int, n_slots: int, kv_dtype: int,
                    host_tier: int = 0, host_grad_dtype: int = PKV_BF16,
                    device_budget_bytes: int = 0, host_grad_accumulate: int = 0,
                    window_slots: int = 0) -> Pool:
    d = pkv_pool_desc(n_layers, n_kv_heads, head_dim, page_size, max_logical_pages, n_slots,
                      kv_dtype, host_tier, host_grad_dtype, host_grad_accumulate,
                      window_slots, device_budget_bytes)
    h = ctypes.c_void_p()
    _check(lib().pkv_pool_create(ctypes.byref(d), ctypes.byref(h)))
    return Pool(h.value, d)


def pkv_pool_destroy(pool: Pool) -> None:
    pool.close()


def pkv_page_table_set(pool: Pool, layer: int, kv_head: int, slots) -> None:
    import numpy as np
    a = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
    _check(lib().pkv_page_table_set(pool.handle, layer, kv_head,
                                    a.ctypes.data_as(ctypes.c_void_p), a.size))


def pkv_length(pool: Pool, layer: int) -> int:
    return int(lib().pkv_length(pool.handle, layer))


def pkv_append_kv(pool: Pool, layer: int, pos0: int, k, v, stream=None) -> None:
    _check(lib().pkv_append_kv(pool.handle, layer, pos0, k.shape[0], _ptr(k), _ptr(v),
                               _stream(stream)))


def pkv_attn_fwd(pool: Pool, layer: int, q_pos0: int, q, o, lse, scale: float,
                 sel=None, stream=None) -> None:
    _check(lib().pkv_attn_fwd(pool.handle, layer, q_pos0, q.shape[0], q.shape[1], scale,
                              _ptr(q), _selp(sel), _ptr(o), _ptr(lse), _stream(stream)))


def pkv_attn_bwd(pool: Pool, layer: int, q_pos0: int, q, o, dout, lse, dq, scale: float,
                 sel=None, stream=None) -> None:
    _check(lib().pkv_attn_bwd(pool.handle, layer, q_pos0, q.shape[0], q.shape[1], scale,
                              _ptr(q), _ptr(o), _ptr(dout), _ptr(lse), _selp(sel), _ptr(dq),
                              _stream(stream)))


def pkv_attn_bwd_noalloc(pool: Pool, layer: int, q_pos0: int, q, o, dout, lse, dq, scale: float,
                         sel=None, stream=None) -> None:
    _check(lib().pkv_attn_bwd_noalloc(pool.handle, layer, q_pos0, q.shape[0], q.shape[1], scale,
                                      _ptr(q), _ptr(o), _ptr(dout), _ptr(lse), _selp(sel),
                                      _ptr(dq), _stream(stream)))


def pkv_select_topk_pages(pool: Pool, layer: int, q_pos0: int, q, top_k: int, sel_pages,
                          sel_count, n_sink: int = 1, n_local: int = 2, stream=None) -> None:
    _check(lib().pkv_select_topk_pages(pool.handle, layer, q_pos0, q.shape[0], q.shape[1],
                                       _ptr(q), top_k, n_sink, n_local, _ptr(sel_pages),
                                       _ptr(sel_count), sel_pages.shape[2], _stream(stream)))


def pkv_prefetch_pages(pool: Pool, layer: int, sel=None, with_grads: bool = False,
                       copy_stream=None, ready=None) -> None:
    ev = None if ready is None else ready.cuda_event
    _check(lib().pkv_prefetch_pages(pool.handle, layer, _selp(sel), int(with_grads),
                                    _stream(copy_stream), ev))


def pkv_prefetch_prefix(pool: Pool, layer: int, n_keys: int, with_grads: bool = False,
                        copy_stream=None, ready=None) -> None:
    ev = None if ready is None else ready.cuda_event
    _check(lib().pkv_prefetch_prefix(pool.handle, layer, n_keys, int(with_grads),
                                     _stream(copy_stream), ev))


def pkv_writeback_grads(pool: Pool, layer: int, copy_stream=None, done=None) -> None:
    ev = None if done is None else done.cuda_event
    _check(lib().pkv_writeback_grads(pool.handle, layer, _stream(copy_stream), ev))


def pkv_grad_zero(pool: Pool, layer: int, stream=None) -> None:
    _check(lib().pkv_grad_zero(pool.handle, layer, _stream(stream)))


def pkv_read_pages(pool: Pool, layer: int, what: int, dst, stream=None) -> None:
    _check(lib().pkv_read_pages(pool.handle, layer, what, _ptr(dst), _stream(stream)))


def pkv_pool_bytes(pool: Pool) -> tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().pkv_pool_bytes(pool.handle, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def pkv_offload_bytes(pool: Pool) -> tuple[int, int]:
    """(bytes fetched host->HBM, bytes written back HBM->host) so far."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().pkv_offload_bytes(pool.handle, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def pkv_pool_reset(pool: Pool, layer: int) -> None:
    _check(lib().pkv_pool_reset(pool.handle, layer))


def pkv_kernel_timing(enable: bool) -> None:
    _check(lib().pkv_kernel_timing(int(enable)))


def pkv_kernel_times() -> dict:
    """{kind: (total_ms, launches)} since timing was enabled."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().pkv_kernel_times(n, ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}


def pkv_read_rows(pool: Pool, layer: int, what: int, pos0: int, dst, stream=None) -> None:
    """Rows [pos0, pos0 + dst.shape[0]) of K, V, dK or dV of `layer`, logical order."""
    _check(lib().pkv_read_rows(pool.handle, layer, what, pos0, dst.shape[0], _ptr(dst),
                               _stream(stream)))


def pkv_measure_gather(pool: Pool, layer: int, q_pos0: int, n_q: int, n_q_heads: int, out,
                       sel=None, stream=None) -> None:
    """Measurement kernel: stream the K/V tiles pkv_attn_fwd would read, no math."""
    _check(lib().pkv_measure_gather(pool.handle, layer, q_pos0, n_q, n_q_heads, _selp(sel),
                                    _ptr(out), _stream(stream)))


def pkv_measure_atomics(pool: Pool, layer: int, n_keys: int, reps: int, value: float = 0.0,
                        stream=None) -> None:
    """Measurement kernel: the dK/dV atomic epilogue over keys [0, n_keys), reps times."""
    _check(lib().pkv_measure_atomics(pool.handle, layer, n_keys, reps, value, _stream(stream)))


def pkv_last_error() -> str:
    msg = lib().pkv_last_error()
    return msg.decode() if msg else ""
