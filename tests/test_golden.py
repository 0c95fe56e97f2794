"""The oracle against the stored expectations in tests/golden/: a
hand-derived worked example (orders) and the recorded plan, stop points and
output checksums of the 2048-token workload (a change of the oracle's
arithmetic shows up here)."""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np
import pytest

import oracle as O
from synthetic import get_config, make_stripe_inputs, round_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def worked_inputs(g, variant, d=None):
    """bf16 bits of the worked example; `d` zero-pads the head dimension."""
    N, d0 = g["N"], g["head_dim"]
    d = d or d0
    qf = np.zeros((1, 1, N, d), np.float32)
    qf[0, 0, :, 0] = g["query"]["coord0_all_rows"]
    qf[0, 0, 128:192, 1] = g["query"]["coord1_rows_128_191"]
    kf = np.zeros((1, 1, N, d), np.float32)
    for j, a in g["key"]["coord0"].items():
        kf[0, 0, int(j), 0] = a
    for j, a in g["key"]["coord1"].items():
        kf[0, 0, int(j), 1] = a
    if variant == "prefix":
        for j, a in g["key"]["coord1_prefix_variant_extra"].items():
            kf[0, 0, int(j), 1] = a
    return round_to_bf16_bits(qf), round_to_bf16_bits(kf)


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).astype(np.int64).tobytes()
                          ).hexdigest()


@pytest.mark.parametrize("variant", ["plain", "prefix"])
def test_worked_orders(variant):
    g = load("worked_orders.json")
    q, k = worked_inputs(g, variant)
    pl = O.plan(q, k, g["segment"])
    exp = g["expected"][variant]
    assert pl.pi_k[0, 0].tolist() == exp["pi_k"]
    for t in (1, 2, 3):
        assert O.restricted_list(pl, 0, 0, t).tolist() == exp[f"L_{t}"]
    assert pl.pi_q[0, 0].tolist() == exp["pi_q"]


def test_tiny_reference():
    ref = load("tiny_n2048_reference.json")
    cfg = get_config(1)
    q, k, v = make_stripe_inputs(cfg.spec)
    pl = O.plan(q, k, ref["segment"])
    for name, h in ref["sha256_int64"].items():
        assert sha(getattr(pl, name)) == h, name
    for tau, r in ref["taus"].items():
        n_I, _ = O.stop_points(q, k, pl, float(tau))
        assert n_I.reshape(-1).tolist() == r["n_I"], tau
        o, lse = O.attend(q, k, v, pl, n_I)
        assert abs(o.sum() - r["o_sum"]) <= 1e-9 * max(1.0, abs(r["o_sum"]))
        assert abs((o * o).sum() - r["o_sumsq"]) <= 1e-9 * r["o_sumsq"]
        assert abs(lse.sum() - r["lse_sum"]) <= 1e-9 * abs(r["lse_sum"])
        assert np.allclose(o[0, 0, :6, :8], r["o_rows_0_5_first8"],
                           rtol=0, atol=1e-12)
