"""Writes the stored expectations under tests/golden/.

worked_orders.json -- a hand-derived example (no oracle call): the expected
  key and query orders follow from the derivation written next to them.
  Pages: S2O page, *Summary* (a global key/value order and a segment-local
  query order ranked by stripe-level mean pooling); AB-Sparse page, the
  block-sparse workflow paragraph and its mean-pooling footnote.
tiny_n2048_reference.json -- the oracle's plan, stop points and output
  checksums on the 2048-token workload, written by calling oracle/ only; a
  later change of the oracle's arithmetic shows up as a mismatch here.

Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).astype(np.int64).tobytes()
                          ).hexdigest()


def worked_orders():
    """N = 256, S = 64, d = 8 (zero-padding to any d changes nothing).

    Queries: every row has 1.0 in coordinate 0; rows 128..191 (segment 2)
    also carry (2 m_i - 63) / 128 in coordinate 1, m = (37 i) mod 64, a
    zero-sum permutation of odd multiples of 1/128, exact in bf16. Keys:
    coordinate 0 is 2.0, 1.5, 1.0, 0.5 at keys 5, 70, 130, 200 and 0
    elsewhere; key 70 has 1.0 in coordinate 1; variant "prefix" also puts
    1.0 in coordinate 1 of keys 100, 101, 102.

    Fixed point (x 256): fx(q_i) = (256, 4 m_i - 126 in segment 2, 0, ...).
    The pooled query is P = (65536, 0, ...) because the coordinate-1 values
    sum to zero. Key scores v_j = 65536 * 256 * a_j: keys 5, 70, 130, 200
    first, in that order; every other key scores 0 and follows in index
    order (ties by index).
    L_t = that order restricted to keys < 64 t, so L_1 = [5, rest of
    0..63], L_2 = [5, 70, rest of 0..127], L_3 = [5, 70, 130, rest of
    0..191].
    Query order, segment 1: its top tile is all of segment 0, which is also
    its whole prefix, so C_1 = 64 * top - 64 * prefix = 0: identity.
    Segment 2: top tile of L_2 = keys 5, 70 and 62 keys of zero coordinate
    1 except key 70; prefix = keys 0..127. Coordinate 1 of
    C_2 = 128 * (256) - 64 * (256 [+ 3 * 256 with the prefix variant]) =
    16384 > 0, or -32768 < 0 with the prefix variant; coordinate 0 is
    equal for all queries of the segment. So u_i is an increasing function
    of m_i (decreasing with the prefix variant): queries sorted by m
    descending (ascending), ties impossible (m is a permutation).
    Segment 3: all its queries equal (256, 0, ...): identity.
    """
    N, S, d = 256, 64, 8
    m = [(37 * i) % 64 for i in range(64)]
    hot = [5, 70, 130, 200]
    rest = [j for j in range(N) if j not in hot]
    out = {"N": N, "segment": S, "head_dim": d,
           "query": {"coord0_all_rows": 1.0,
                     "coord1_rows_128_191": [(2 * x - 63) / 128.0 for x in m]},
           "key": {"coord0": {"5": 2.0, "70": 1.5, "130": 1.0, "200": 0.5},
                   "coord1": {"70": 1.0},
                   "coord1_prefix_variant_extra": {"100": 1.0, "101": 1.0,
                                                   "102": 1.0}},
           "expected": {}}
    for variant in ("plain", "prefix"):
        local = sorted(range(64), key=(lambda i: m[i]) if variant == "prefix"
                       else (lambda i: -m[i]))
        out["expected"][variant] = {
            "pi_k": hot + rest,
            "L_1": [5] + [j for j in range(64) if j != 5],
            "L_2": [5, 70] + [j for j in range(128) if j not in (5, 70)],
            "L_3": [5, 70, 130] + [j for j in range(192)
                                   if j not in (5, 70, 130)],
            "pi_q": list(range(128)) + [128 + i for i in local]
            + list(range(192, 256)),
        }
    out["derivation"] = worked_orders.__doc__
    out["citation"] = ("S2O page, Summary (global key/value order and "
                       "segment-local query order by stripe-level mean "
                       "pooling); AB-Sparse page, block-sparse workflow "
                       "paragraph (mean-pooled block representatives)")
    return out


def tiny_reference():
    import oracle as O
    from synthetic import get_config, make_stripe_inputs
    cfg = get_config(1)
    q, k, v = make_stripe_inputs(cfg.spec)
    S = cfg.segment
    pl = O.plan(q, k, S)
    ref = {"workload": cfg.name, "segment": S,
           "sha256_int64": {"pi_k": sha(pl.pi_k), "pi_q": sha(pl.pi_q),
                            "L": sha(pl.L), "key_score": sha(pl.key_score),
                            "query_score": sha(pl.query_score),
                            "contrast": sha(pl.contrast)},
           "taus": {}}
    for tau in (0.005, 0.05, 0.2):
        n_I, _ = O.stop_points(q, k, pl, tau)
        o, lse = O.attend(q, k, v, pl, n_I)
        ref["taus"][repr(tau)] = {
            "n_I": n_I.reshape(-1).tolist(),
            "o_sum": float(o.sum()), "o_sumsq": float((o * o).sum()),
            "lse_sum": float(lse.sum()),
            "o_rows_0_5_first8": o[0, 0, :6, :8].tolist(),
        }
    return ref


def main():
    with open(os.path.join(HERE, "worked_orders.json"), "w") as f:
        json.dump(worked_orders(), f, indent=1)
    with open(os.path.join(HERE, "tiny_n2048_reference.json"), "w") as f:
        json.dump(tiny_reference(), f, indent=1)
    print("wrote", HERE)


if __name__ == "__main__":
    main()
