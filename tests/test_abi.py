"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments with the documented status codes before launching anything (these
calls make no GPU work, so they run on the CPU)."""
import ctypes
import os
import re

import pytest

from permuted_block_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libsparse_attn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) == 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED_SYMBOLS)


def P(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, seq_len=1024, head_dim=128,
                segment=256, block=64, tau=0.01, flags=0)
    base.update(kw)
    return _lib.SaParams(**base)


def ws(p):
    return _lib.load().sparse_attn_workspace_bytes(ctypes.byref(p))


def test_workspace_bytes_valid_and_invalid():
    assert ws(P()) > 0
    assert ws(P(seq_len=131072, heads_q=32, heads_kv=8, segment=2048)) > 0
    bad = [dict(block=32), dict(head_dim=64), dict(segment=96),
           dict(seq_len=1000), dict(seq_len=262144, segment=2048),
           dict(heads_q=3), dict(tau=-1.0), dict(tau=float("nan")),
           dict(tau=float("inf")), dict(batch=0), dict(flags=64)]
    for kw in bad:
        assert ws(P(**kw)) == 0, kw


def test_plan_rejects_before_launch():
    lib = _lib.load()
    out = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)    # never dereferenced: rejected first
    p = P()
    n = ws(p)
    call = lambda p_, q, k, w, nbytes: lib.sparse_attn_plan(
        ctypes.byref(p_) if p_ is not None else None, q, k, w, nbytes, None,
        ctypes.byref(out))
    assert call(None, fake, fake, fake, n) == _lib.SA_ERR_NULL_POINTER
    assert call(p, None, fake, fake, n) == _lib.SA_ERR_NULL_POINTER
    assert call(p, fake, fake, None, n) == _lib.SA_ERR_NULL_POINTER
    assert call(p, fake, fake, fake, n - 1) == _lib.SA_ERR_WORKSPACE_TOO_SMALL
    assert call(p, fake, fake, ctypes.c_void_p((1 << 20) + 8), n) == \
        _lib.SA_ERR_INVALID_ARG
    assert call(P(segment=100), fake, fake, fake, n) == \
        _lib.SA_ERR_UNSUPPORTED_SHAPE
    assert call(P(tau=-0.5), fake, fake, fake, n) == _lib.SA_ERR_INVALID_ARG
    assert out.value is None
    assert lib.sparse_attn_plan(ctypes.byref(p), fake, fake, fake, n, None,
                                None) == _lib.SA_ERR_NULL_POINTER


def test_forward_rejects_before_launch():
    """sparse_attn_forward checks its own arguments and the plan's before it
    enqueues anything."""
    lib = _lib.load()
    f = ctypes.c_void_p(1 << 20)
    p = P()
    n = lib.sparse_attn_workspace_bytes(ctypes.byref(p))
    out = ctypes.c_void_p()
    assert lib.sparse_attn_forward(ctypes.byref(p), f, f, f, f, None, f, n,
                                   None, None, None) == \
        _lib.SA_ERR_NULL_POINTER
    for args in ((f, f, None, f), (f, f, f, None), (None, f, f, f)):
        assert lib.sparse_attn_forward(ctypes.byref(p), *args, None, f, n,
                                       None, None, ctypes.byref(out)) == \
            _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_forward(ctypes.byref(p), f, f, f, f, None, f,
                                   n - 1, None, None, ctypes.byref(out)) == \
        _lib.SA_ERR_WORKSPACE_TOO_SMALL
    assert out.value is None


def test_forward_static_rejects_before_launch():
    """The entry point without allocation rejects null pointers, invalid
    shapes and shapes whose workspace exceeds its fixed scratch before it
    touches the GPU."""
    lib = _lib.load()
    f = ctypes.c_void_p(1 << 20)
    p = P()
    assert ws(p) <= _lib.SA_STATIC_SCRATCH_BYTES
    call = lambda p_, *a: lib.sparse_attn_forward_static(
        ctypes.byref(p_) if p_ is not None else None, *a, None, None)
    assert call(None, f, f, f, f) == _lib.SA_ERR_NULL_POINTER
    for args in ((None, f, f, f), (f, None, f, f), (f, f, None, f),
                 (f, f, f, None)):
        assert call(p, *args) == _lib.SA_ERR_NULL_POINTER
    assert call(P(segment=100), f, f, f, f) == _lib.SA_ERR_UNSUPPORTED_SHAPE
    assert call(P(tau=-1.0), f, f, f, f) == _lib.SA_ERR_INVALID_ARG
    big = P(heads_q=32, heads_kv=8, seq_len=32768, segment=2048)
    assert ws(big) > _lib.SA_STATIC_SCRATCH_BYTES
    assert call(big, f, f, f, f) == _lib.SA_ERR_WORKSPACE_TOO_SMALL


def test_other_entry_points_reject_null():
    lib = _lib.load()
    f = ctypes.c_void_p(1 << 20)
    assert lib.sparse_attn_prefill(None, f, f, f, f, None, None) == \
        _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_plan_set_tau(None, 0.1) == _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_plan_set_kv_order(None, f, None) == \
        _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_plan_export(None, 0, f, 8, None) == \
        _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_plan_export_bytes(None, 0) == 0
    assert lib.sparse_attn_plan_set_topk(None, 3, f, 8, None) == \
        _lib.SA_ERR_NULL_POINTER
    assert lib.sparse_attn_topk_scratch_bytes(None) == 0
    lib.sparse_attn_plan_destroy(None)


def test_status_strings():
    lib = _lib.load()
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = lib.sparse_attn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.sparse_attn_status_string(-99).decode() == "unknown status"
