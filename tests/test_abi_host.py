"""CPU checks of the C ABI: the library loads and exports every entry point
include/pkv.h declares, and the binding wraps each of them (no compute)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_chunk_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = _declared()
    for n in ("pkv_pool_create", "pkv_append_kv", "pkv_attn_fwd", "pkv_attn_bwd",
              "pkv_select_topk_pages", "pkv_prefetch_pages"):
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("libpkv.so not built")
    L = ctypes.CDLL(pkv.LIB_PATH)
    for n in _declared():
        assert hasattr(L, n), n


def test_binding_wraps_every_declared_symbol():
    names = _declared()
    assert sorted(pkv.EXPORTS) == names
    for n in names:
        assert callable(getattr(pkv, n)), n


def test_binding_loads_signatures():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("libpkv.so not built")
    L = pkv.lib()
    assert L.pkv_attn_fwd.argtypes is not None
    assert pkv.pkv_last_error() == ""
