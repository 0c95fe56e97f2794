"""GPU: the stop points are scanned from pooled means by the plan and
rescanned by the next prefill after any setter; the attention kernel stops
every block at them. Compared with the CPU oracle's stop points (up to
documented near-tau ties) and, where the selection is the same, with the
GPU's own earlier results bit for bit."""
import numpy as np
import pytest

import oracle as O
from synthetic import StripeSpec, make_stripe_inputs
from tests.gpu_helpers import (assert_outputs_close, bf16_tensor_to_f64, say,
                               stop_mismatches, to_device)

pytestmark = pytest.mark.gpu


def _inputs(seed, N=1024, Hq=4, Hkv=2):
    spec = StripeSpec(1, Hq, Hkv, N, 128, n_vert=16, n_horiz=8, window=64,
                      seed=seed)
    return make_stripe_inputs(spec)


def _prefill(pbs, pl, tq, tk, tv):
    import torch
    o, lse = pbs.prefill(pl, tq, tk, tv, return_lse=True)
    torch.cuda.synchronize()
    return bf16_tensor_to_f64(o), lse.cpu().numpy().astype(np.float64)


def test_stop_points_after_plan():
    """n_I right after the plan call (no prefill yet) equals the oracle's."""
    import permuted_block_sparse_amd as pbs
    q, k, v = _inputs(50)
    S = 256
    pl_o = O.plan(q, k, S)
    for tau in (0.02, 0.1, 1.5):
        say(f"[stops] after plan, tau={tau}")
        pl = pbs.plan(to_device(q), to_device(k), S, tau)
        n_gpu = pl.n_I()
        n_orc, traces = O.stop_points(q, k, pl_o, tau)
        stop_mismatches(n_gpu, n_orc, traces, tau)
        if tau >= 1.0:   # the share of any tile is <= 1: stop at k = 0
            assert (n_gpu == 0).all()


def test_setters_rescan():
    """set_tau / set_budget / set_max_threshold take effect on the next
    prefill, and returning to an earlier setting gives the earlier stop
    points and bit-identical outputs."""
    import permuted_block_sparse_amd as pbs
    q, k, v = _inputs(51)
    S = 256
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    pl_o = O.plan(q, k, S)
    pl = pbs.plan(tq, tk, S, 0.02)
    say("[stops] tau 0.02")
    o1, l1 = _prefill(pbs, pl, tq, tk, tv)
    n1 = pl.n_I().copy()
    say("[stops] set_tau 0.2")
    pl.set_tau(0.2)
    o2, l2 = _prefill(pbs, pl, tq, tk, tv)
    n2 = pl.n_I()
    n_orc, traces = O.stop_points(q, k, pl_o, 0.2)
    ties = stop_mismatches(n2, n_orc, traces, 0.2)
    n_use = n_orc.copy()
    for b, h, I in ties:
        n_use[b, h, I] = n2[b, h, I]
    o_ref, l_ref = O.attend(q, k, v, pl_o, n_use)
    assert_outputs_close(o2, o_ref, l2, l_ref)
    assert (n2 <= n1).all() and (n2 < n1).any()
    say("[stops] set_budget 3, then -1")
    pl.set_budget(3)
    _prefill(pbs, pl, tq, tk, tv)
    nb = pl.n_I()
    t = np.arange(nb.shape[-1]) * 64 // S
    assert np.array_equal(nb, np.broadcast_to(np.minimum(3, t * S // 64),
                                              nb.shape))
    pl.set_budget(-1)
    pl.set_tau(0.02)
    o3, l3 = _prefill(pbs, pl, tq, tk, tv)
    assert np.array_equal(pl.n_I(), n1)
    assert np.array_equal(o3, o1) and np.array_equal(l3, l1)
    say("[stops] exact max test, then back to the tau stop")
    pl.set_max_threshold(-np.inf)
    od, ld = _prefill(pbs, pl, tq, tk, tv)
    assert np.array_equal(pl.n_I(), np.broadcast_to(t * S // 64, nb.shape))
    o_dense, l_dense = O.dense_causal(q, k, v)
    assert_outputs_close(od, o_dense, ld, l_dense)
    pl.set_max_threshold(float("nan"))
    o4, l4 = _prefill(pbs, pl, tq, tk, tv)
    assert np.array_equal(pl.n_I(), n1)
    assert np.array_equal(o4, o1) and np.array_equal(l4, l1)


def test_kv_order_injection_rescans():
    """After set_kv_order the stop points follow the new lists."""
    import torch
    import permuted_block_sparse_amd as pbs
    q, k, v = _inputs(52, N=768, Hq=2, Hkv=1)
    S = 128
    perm = np.random.default_rng(52).permutation(768)[None, None]
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    pl = pbs.plan(tq, tk, S, 0.05)
    say("[stops] injected KV order")
    pl.set_kv_order(torch.from_numpy(
        np.ascontiguousarray(perm, dtype=np.int32)).to("cuda:0"))
    n_after = pl.n_I()
    pl_o = O.plan(q, k, S, kv_order=perm)
    n_orc, traces = O.stop_points(q, k, pl_o, 0.05)
    stop_mismatches(n_after, n_orc, traces, 0.05)
    o, lse = _prefill(pbs, pl, tq, tk, tv)
    assert np.array_equal(pl.n_I(), n_after)
    n_use = n_orc.copy()
    for b, h, I in np.argwhere(n_after != n_orc):
        n_use[b, h, I] = n_after[b, h, I]
    o_ref, l_ref = O.attend(q, k, v, pl_o, n_use)
    assert_outputs_close(o, o_ref, lse, l_ref)
