"""Permuted, early-stopping block-sparse causal prefill attention on MI355X.

Thin Python binding over libsparse_attn.so (include/sparse_attn.h). torch is
used only to own device memory and to supply the current HIP stream; every
step of the computation runs in the library's gfx950 kernels. There is no
CPU fallback: without the built library every call raises.

    pl = plan(q, k, segment=2048, tau=0.005)    # estimator + index builder
    o = prefill(pl, q, k, v)                    # gather attention + stop
    o, lse = prefill(pl, q, k, v, return_lse=True)

q: [B, Hq, N, 128] bfloat16 CUDA tensor; k, v: [B, Hkv, N, 128].
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import (SA_NO_QPERM, SA_NO_KVPERM, SA_NO_EARLYSTOP,
                   SA_LOCAL_ONLY, SA_SEGMENT_KV, SparseAttnError)

__all__ = ["plan", "prefill", "forward", "forward_static", "SparsePlan",
           "SA_NO_QPERM",
           "SA_NO_KVPERM",
           "SA_NO_EARLYSTOP", "SA_LOCAL_ONLY", "SA_SEGMENT_KV",
           "SparseAttnError",
           "workspace_bytes"]

_EXPORT_DTYPES = {
    _lib.SA_EXPORT_PI_K: np.int32, _lib.SA_EXPORT_PI_Q: np.int32,
    _lib.SA_EXPORT_L: np.int32, _lib.SA_EXPORT_N_I: np.int32,
    _lib.SA_EXPORT_KEY_SCORE: np.int64, _lib.SA_EXPORT_QUERY_SCORE: np.int64,
    _lib.SA_EXPORT_CONTRAST: np.int64, _lib.SA_EXPORT_POOLED: np.int64,
    _lib.SA_EXPORT_TOPK_MASK: np.uint32,
}


def _stream_of(stream: Optional[torch.cuda.Stream]) -> torch.cuda.Stream:
    return stream if stream is not None else torch.cuda.current_stream()


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    return _stream_of(stream).cuda_stream


def _record(tensors, streams) -> None:
    """Tell torch's caching allocator that work enqueued on `streams` uses
    `tensors`: memory freed on the host side is not handed out again before
    that work has completed (the library's kernels run on the caller's
    streams, not necessarily torch's current one)."""
    for s in streams:
        for t in tensors:
            if t is not None:
                t.record_stream(s)


def _check_tensor(x: torch.Tensor, name: str, heads_dim_ok=True):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 4-D tensor")


def _params(q, k, segment, tau, block, flags) -> _lib.SaParams:
    B, Hq, N, d = q.shape
    return _lib.SaParams(B, Hq, k.shape[1], N, d, segment, block, float(tau),
                         int(flags))


def workspace_bytes(batch, heads_q, heads_kv, seq_len, segment, head_dim=128,
                    block=64, tau=0.0, flags=0) -> int:
    lib = _lib.load()
    p = _lib.SaParams(batch, heads_q, heads_kv, seq_len, head_dim, segment,
                      block, float(tau), int(flags))
    return int(lib.sparse_attn_workspace_bytes(ctypes.byref(p)))


class SparsePlan:
    """A plan (index arrays in a device workspace owned by this object)."""

    def __init__(self, q, k, segment, tau, block=64, flags=0, stream=None,
                 _launch=None):
        lib = _lib.load()
        _check_tensor(q, "q")
        _check_tensor(k, "k")
        if q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
            raise ValueError("q and k shapes do not agree")
        self.params = _params(q, k, segment, tau, block, flags)
        nbytes = lib.sparse_attn_workspace_bytes(ctypes.byref(self.params))
        if nbytes == 0:
            raise SparseAttnError(_lib.SA_ERR_UNSUPPORTED_SHAPE,
                                  "sparse_attn_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8,
                                     device=q.device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self._handle = ctypes.c_void_p()
        self.shape = tuple(q.shape)
        self.heads_kv = k.shape[1]
        self._inputs = (q, k)   # the plan keeps device pointers to both
        if _launch is None:
            st = lib.sparse_attn_plan(
                ctypes.byref(self.params), ctypes.c_void_p(q.data_ptr()),
                ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(self._ws_ptr),
                ctypes.c_size_t(nbytes), ctypes.c_void_p(_stream_ptr(stream)),
                ctypes.byref(self._handle))
            _lib.check(st, "sparse_attn_plan")
            self.used_on(stream)
        else:  # a call that builds the plan itself (sparse_attn_forward)
            _launch(self, nbytes)

    def used_on(self, *streams) -> None:
        """Record the workspace (and the inputs the plan points to) on the
        streams whose enqueued work uses them."""
        _record((self.workspace,) + self._inputs,
                [_stream_of(s) for s in streams])

    @property
    def tau(self) -> float:
        return self.params.tau

    def set_tau(self, tau: float) -> None:
        _lib.check(_lib.load().sparse_attn_plan_set_tau(self._handle,
                                                        float(tau)),
                   "sparse_attn_plan_set_tau")
        self.params.tau = float(tau)

    def set_budget(self, tiles: int) -> None:
        """Fixed tile budget per query block instead of the tau stop
        (tiles < 0: back to the tau stop)."""
        _lib.check(_lib.load().sparse_attn_plan_set_budget(self._handle,
                                                           int(tiles)),
                   "sparse_attn_plan_set_budget")

    def set_max_threshold(self, theta: float) -> None:
        """Exact per-block maximum test with threshold theta on the scaled
        logits instead of the tau stop (NaN: back to the tau stop)."""
        _lib.check(_lib.load().sparse_attn_plan_set_max_threshold(
            self._handle, float(theta)), "sparse_attn_plan_set_max_threshold")

    def set_topk(self, tiles: int, stream=None) -> None:
        """Per-block centroid Top-K selection of `tiles` tiles of L_t
        instead of the tau stop (tiles < 0: back to the tau stop). The
        scores' scratch is allocated here for the work this call enqueues
        and released when it has run."""
        lib = _lib.load()
        if tiles < 0:
            _lib.check(lib.sparse_attn_plan_set_topk(
                self._handle, int(tiles), None, 0,
                ctypes.c_void_p(_stream_ptr(stream))),
                "sparse_attn_plan_set_topk")
            return
        n = int(lib.sparse_attn_topk_scratch_bytes(self._handle))
        s = _stream_of(stream)
        with torch.cuda.stream(s):
            scratch = torch.empty(max(n, 8), dtype=torch.uint8,
                                  device=self.workspace.device)
        _lib.check(lib.sparse_attn_plan_set_topk(
            self._handle, int(tiles), ctypes.c_void_p(scratch.data_ptr()),
            ctypes.c_size_t(n), ctypes.c_void_p(s.cuda_stream)),
            "sparse_attn_plan_set_topk")
        self.used_on(stream)
        _record((scratch,), [s])

    def topk_masks(self):
        """Selected tiles of every block after set_topk: uint32
        [B, Hq, N / 64, 64], bit p of word w = position 32 w + p of L_t."""
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_TOPK_MASK).reshape(B, Hq, N // 64,
                                                             64)

    def set_kv_order(self, pi_k: torch.Tensor, stream=None) -> None:
        if pi_k.dtype != torch.int32 or not pi_k.is_cuda:
            raise TypeError("pi_k must be an int32 CUDA tensor")
        B, Hq, N, _ = self.shape
        if tuple(pi_k.shape) != (B, self.heads_kv, N):
            raise ValueError("pi_k must be [B, Hkv, N]")
        pi_k = pi_k.contiguous()
        _lib.check(_lib.load().sparse_attn_plan_set_kv_order(
            self._handle, ctypes.c_void_p(pi_k.data_ptr()),
            ctypes.c_void_p(_stream_ptr(stream))),
            "sparse_attn_plan_set_kv_order")
        self._keepalive = pi_k
        self.used_on(stream)
        _record((pi_k,), [_stream_of(stream)])

    def export(self, what: int, stream=None) -> np.ndarray:
        lib = _lib.load()
        n = lib.sparse_attn_plan_export_bytes(self._handle, what)
        dt = _EXPORT_DTYPES[what]
        out = np.empty(n // np.dtype(dt).itemsize, dtype=dt)
        if n:
            _lib.check(lib.sparse_attn_plan_export(
                self._handle, what, out.ctypes.data_as(ctypes.c_void_p), n,
                ctypes.c_void_p(_stream_ptr(stream))),
                "sparse_attn_plan_export")
        return out

    def pi_k(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_PI_K).reshape(B, self.heads_kv, N)

    def pi_q(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_PI_Q).reshape(B, Hq, N)

    def n_I(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_N_I).reshape(B, Hq, N // 64)

    def restricted_lists(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_L).reshape(B, self.heads_kv, -1)

    def key_score(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_KEY_SCORE).reshape(
            B, self.heads_kv, N)

    def query_score(self):
        B, Hq, N, _ = self.shape
        return self.export(_lib.SA_EXPORT_QUERY_SCORE).reshape(B, Hq, N)

    def contrast(self):
        B, Hq, N, _ = self.shape
        T = N // self.params.segment
        return self.export(_lib.SA_EXPORT_CONTRAST).reshape(
            B, self.heads_kv, T, 128)

    def pooled(self):
        B = self.shape[0]
        return self.export(_lib.SA_EXPORT_POOLED).reshape(B, self.heads_kv,
                                                          128)

    def close(self) -> None:
        if getattr(self, "_handle", None) and self._handle.value:
            _lib.load().sparse_attn_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan(q: torch.Tensor, k: torch.Tensor, segment: int, tau: float,
         block: int = 64, flags: int = 0, stream=None) -> SparsePlan:
    """Importance estimation and index building (sparse_attn_plan)."""
    return SparsePlan(q, k, segment, tau, block, flags, stream)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, segment: int,
            tau: float, block: int = 64, flags: int = 0,
            out: Optional[torch.Tensor] = None, return_lse: bool = False,
            stream=None, side_stream=None):
    """Plan and prefill in one call (sparse_attn_forward): the dense local
    windows run on `side_stream` (a second stream of the same device; None:
    the plan and the attention one after the other on `stream`) while the
    planner runs on `stream`. Returns (plan, o) or (plan, o, lse); the plan
    serves the setters, exports and later prefills as from plan()."""
    lib = _lib.load()
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(x, n)
    if k.shape != v.shape:
        raise ValueError("k and v shapes do not agree")
    o = out if out is not None else torch.empty_like(q)
    _check_tensor(o, "out")
    lse = (torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
           if return_lse else None)
    main = _stream_ptr(stream)
    side = _stream_ptr(side_stream) if side_stream is not None else main
    streams = [_stream_of(stream)] + (
        [side_stream] if side_stream is not None else [])

    def launch(pl, nbytes):
        st = lib.sparse_attn_forward(
            ctypes.byref(pl.params), ctypes.c_void_p(q.data_ptr()),
            ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(o.data_ptr()),
            ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
            ctypes.c_void_p(pl._ws_ptr), ctypes.c_size_t(nbytes),
            ctypes.c_void_p(main), ctypes.c_void_p(side),
            ctypes.byref(pl._handle))
        _lib.check(st, "sparse_attn_forward")
        pl.used_on(*streams)
        _record((v, o, lse), streams)

    pl = SparsePlan(q, k, segment, tau, block, flags, stream, _launch=launch)
    return (pl, o, lse) if return_lse else (pl, o)


def forward_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   segment: int, tau: float, block: int = 64, flags: int = 0,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None):
    """Plan and prefill on one stream with the library's fixed device
    scratch (sparse_attn_forward_static): no workspace and no plan object;
    the library allocates nothing. Pass `out` (and `lse`) to allocate
    nothing here either. Shapes whose workspace exceeds
    SA_STATIC_SCRATCH_BYTES are rejected. Calls that overlap on one GPU
    race. Returns o, or (o, lse) when lse is given."""
    lib = _lib.load()
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(x, n)
    if k.shape != v.shape:
        raise ValueError("k and v shapes do not agree")
    o = out if out is not None else torch.empty_like(q)
    _check_tensor(o, "out")
    params = _params(q, k, segment, tau, block, flags)
    st = lib.sparse_attn_forward_static(
        ctypes.byref(params), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
        ctypes.c_void_p(_stream_ptr(stream)))
    _lib.check(st, "sparse_attn_forward_static")
    _record((q, k, v, o, lse), [_stream_of(stream)])
    return (o, lse) if lse is not None else o


def prefill(pl: SparsePlan, q: torch.Tensor, k: torch.Tensor,
            v: torch.Tensor, out: Optional[torch.Tensor] = None,
            return_lse: bool = False, stream=None):
    """Gather attention with the tau stop (sparse_attn_prefill)."""
    lib = _lib.load()
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(x, n)
    if tuple(q.shape) != pl.shape or k.shape != v.shape:
        raise ValueError("q/k/v shapes do not match the plan")
    o = out if out is not None else torch.empty_like(q)
    _check_tensor(o, "out")
    lse = (torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
           if return_lse else None)
    st = lib.sparse_attn_prefill(
        pl._handle, ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
        ctypes.c_void_p(_stream_ptr(stream)))
    _lib.check(st, "sparse_attn_prefill")
    pl.used_on(stream)
    _record((q, k, v, o, lse), [_stream_of(stream)])
    return (o, lse) if return_lse else o
