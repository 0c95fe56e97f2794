"""ctypes declarations of libsparse_attn.so (see include/sparse_attn.h)."""
from __future__ import annotations

import ctypes
import os

# SPARSE_ATTN_LIB names another build of the library (the tests' sanitized
# host build); by default the in-tree one
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED_SHAPE = -2
SA_ERR_WORKSPACE_TOO_SMALL = -3
SA_ERR_HIP = -4
SA_ERR_NULL_POINTER = -5
SA_ERR_HOST_ALLOC = -6

SA_STATIC_SCRATCH_BYTES = 256 << 20  # scratch of sparse_attn_forward_static

SA_NO_QPERM = 1
SA_NO_KVPERM = 2
SA_NO_EARLYSTOP = 4
SA_LOCAL_ONLY = 8
SA_SEGMENT_KV = 16

SA_EXPORT_PI_K = 0
SA_EXPORT_PI_Q = 1
SA_EXPORT_L = 2
SA_EXPORT_N_I = 3
SA_EXPORT_KEY_SCORE = 4
SA_EXPORT_QUERY_SCORE = 5
SA_EXPORT_CONTRAST = 6
SA_EXPORT_POOLED = 7
SA_EXPORT_TOPK_MASK = 8

EXPORTED_SYMBOLS = (
    "sparse_attn_workspace_bytes", "sparse_attn_plan", "sparse_attn_prefill",
    "sparse_attn_forward", "sparse_attn_forward_static",
    "sparse_attn_plan_set_tau", "sparse_attn_plan_set_budget",
    "sparse_attn_plan_set_max_threshold",
    "sparse_attn_topk_scratch_bytes", "sparse_attn_plan_set_topk",
    "sparse_attn_plan_export_bytes",
    "sparse_attn_plan_export", "sparse_attn_plan_set_kv_order",
    "sparse_attn_plan_destroy", "sparse_attn_status_string",
)


class SaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("segment", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("tau", ctypes.c_double),
        ("flags", ctypes.c_uint32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m permuted_block_sparse_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER(SaParams)
    lib.sparse_attn_workspace_bytes.argtypes = [P]
    lib.sparse_attn_workspace_bytes.restype = sz
    lib.sparse_attn_plan.argtypes = [P, vp, vp, vp, sz, vp,
                                     ctypes.POINTER(vp)]
    lib.sparse_attn_plan.restype = i32
    lib.sparse_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.sparse_attn_prefill.restype = i32
    lib.sparse_attn_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, vp,
                                        ctypes.POINTER(vp)]
    lib.sparse_attn_forward.restype = i32
    lib.sparse_attn_forward_static.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sparse_attn_forward_static.restype = i32
    lib.sparse_attn_plan_set_tau.argtypes = [vp, ctypes.c_double]
    lib.sparse_attn_plan_set_tau.restype = i32
    lib.sparse_attn_plan_set_budget.argtypes = [vp, i32]
    lib.sparse_attn_plan_set_budget.restype = i32
    lib.sparse_attn_plan_set_max_threshold.argtypes = [vp, ctypes.c_double]
    lib.sparse_attn_plan_set_max_threshold.restype = i32
    lib.sparse_attn_topk_scratch_bytes.argtypes = [vp]
    lib.sparse_attn_topk_scratch_bytes.restype = sz
    lib.sparse_attn_plan_set_topk.argtypes = [vp, i32, vp, sz, vp]
    lib.sparse_attn_plan_set_topk.restype = i32
    lib.sparse_attn_plan_export_bytes.argtypes = [vp, i32]
    lib.sparse_attn_plan_export_bytes.restype = sz
    lib.sparse_attn_plan_export.argtypes = [vp, i32, vp, sz, vp]
    lib.sparse_attn_plan_export.restype = i32
    lib.sparse_attn_plan_set_kv_order.argtypes = [vp, vp, vp]
    lib.sparse_attn_plan_set_kv_order.restype = i32
    lib.sparse_attn_plan_destroy.argtypes = [vp]
    lib.sparse_attn_plan_destroy.restype = None
    lib.sparse_attn_status_string.argtypes = [i32]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = load().sparse_attn_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def check(status: int, what: str) -> None:
    if status != SA_OK:
        raise SparseAttnError(status, what)
