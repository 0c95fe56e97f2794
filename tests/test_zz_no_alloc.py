"""The entry point that allocates nothing (sparse_attn_forward_static,
for callers that cannot allocate device memory): through the C ABI, its
outputs equal those of sparse_attn_forward (plan and prefill on one stream)
bit for bit, on two calls in a row, the second with a smaller input, which
reuses the library's fixed scratch."""
import ctypes

import numpy as np
import pytest

from synthetic import StripeSpec, make_stripe_inputs
from tests.gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


def _static(lib, _lib, q, k, v, S, tau, flags=0):
    import torch
    B, Hq, N, d = q.shape
    p = _lib.SaParams(B, Hq, k.shape[1], N, d, S, 64, tau, flags)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    st = lib.sparse_attn_forward_static(
        ctypes.byref(p), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.SA_OK, st
    return o, lse


def test_forward_static_matches_forward():
    import torch
    import permuted_block_sparse_amd as pbs
    from permuted_block_sparse_amd import _lib
    lib = _lib.load()
    cases = [
        # larger first, then a smaller one over the same scratch
        ("b1_h8_kv2_n8192_s1024", StripeSpec(1, 8, 2, 8192, 128, n_vert=32,
                                             n_horiz=8, window=128, seed=61),
         1024, 0.02, 0),
        ("b2_h4_kv1_n2048_s256", StripeSpec(2, 4, 1, 2048, 128, n_vert=16,
                                            n_horiz=8, window=64, seed=62),
         256, 0.05, pbs.SA_SEGMENT_KV),
    ]
    for name, spec, S, tau, flags in cases:
        q, k, v = make_stripe_inputs(spec)
        tq, tk, tv = to_device(q), to_device(k), to_device(v)
        p = _lib.SaParams(spec.batch, spec.heads_q, spec.heads_kv,
                          spec.seq_len, 128, S, 64, tau, flags)
        assert lib.sparse_attn_workspace_bytes(ctypes.byref(p)) <= \
            _lib.SA_STATIC_SCRATCH_BYTES
        say(f"[no alloc] {name}")
        o_s, l_s = _static(lib, _lib, tq, tk, tv, S, tau, flags)
        torch.cuda.synchronize()
        _, o_f, l_f = pbs.forward(tq, tk, tv, S, tau, flags=flags,
                                  return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_s.view(torch.int16), o_f.view(torch.int16))
        assert torch.equal(l_s, l_f)
        assert torch.isfinite(l_s).all()
        say(f"   equal; mean |o| {float(o_s.float().abs().mean()):.4f}")
