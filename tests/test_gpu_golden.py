"""The HIP path against the stored expectations in tests/golden/, without
running the oracle: the hand-derived worked orders (head dimension
zero-padded to 128, which changes no score) and the recorded plan hashes and
stop points of the 2048-token workload."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_helpers import run_gpu, say
from synthetic import get_config, make_stripe_inputs
from tests.test_golden import load, sha, worked_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["plain", "prefix"])
def test_gpu_worked_orders(variant):
    g = load("worked_orders.json")
    say(f"[golden] worked orders {variant}")
    q, k = worked_inputs(g, variant, d=128)
    v = np.zeros_like(q)
    r = run_gpu(q, k, v, g["segment"], 0.0)
    exp = g["expected"][variant]
    assert r["pi_k"][0, 0].tolist() == exp["pi_k"]
    L = r["L"][0, 0]
    S = g["segment"]
    for t in (1, 2, 3):
        off = S * t * (t - 1) // 2
        assert L[off: off + t * S].tolist() == exp[f"L_{t}"]
    assert r["pi_q"][0, 0].tolist() == exp["pi_q"]


def test_gpu_tiny_reference():
    ref = load("tiny_n2048_reference.json")
    cfg = get_config(1)
    q, k, v = make_stripe_inputs(cfg.spec)
    for tau, rt in ref["taus"].items():
        say(f"[golden] tiny_n2048 tau={tau}")
        r = run_gpu(q, k, v, ref["segment"], float(tau))
        for name in ("pi_k", "pi_q", "L", "key_score", "query_score",
                     "contrast"):
            assert sha(r[name]) == ref["sha256_int64"][name], name
        assert r["n_I"].reshape(-1).tolist() == rt["n_I"], tau
        o = r["o"]
        # bf16 outputs against the oracle's float64 checksums
        assert abs(o.sum() - rt["o_sum"]) <= 2e-3 * o.size ** 0.5 + 1e-2
        assert abs((o * o).sum() - rt["o_sumsq"]) <= 1e-3 * rt["o_sumsq"]
        assert np.abs(o[0, 0, :6, :8] - np.array(rt["o_rows_0_5_first8"])
                      ).max() <= 2e-2
