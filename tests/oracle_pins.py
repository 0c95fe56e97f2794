"""Pins of the CPU oracle, written as functions of the oracle module.

Each ``check_*`` takes the oracle module (``oracle.s2o``, or a copy of it
with a planted mistake) and raises AssertionError when the module disagrees
with what the pages or the mathematics fix. ``test_oracle_pins.py`` runs them
on the real oracle (all must pass); ``test_oracle_mutations.py`` runs them on
copies with planted mistakes (each mistake must make one of them fail).

None of these checks re-types the oracle's own formulas: they use closed
forms, brute-force reformulations, worked examples with hand-derived
answers, library routines, and invariants stated on the pages.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction

import numpy as np
import torch

from synthetic import StripeSpec, make_stripe_inputs, round_to_bf16_bits


def bits(x):
    return round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _rng(seed=7):
    return np.random.Generator(np.random.PCG64(seed))


def _stripe(B=1, Hq=2, Hkv=1, N=512, d=64, seed=11, **kw):
    spec = StripeSpec(B, Hq, Hkv, N, d, n_vert=kw.get("n_vert", 8),
                      n_horiz=kw.get("n_horiz", 4),
                      window=kw.get("window", 32), seed=seed)
    return make_stripe_inputs(spec)


# ---------------------------------------------------------------- inputs

def check_fixed_point(O):
    # 256 x rounded half to even, saturated to int16
    vals = [1.0, -1.0, 0.5, 2.0 ** -9, 3 * 2.0 ** -9, 5 * 2.0 ** -9,
            -3 * 2.0 ** -9, 200.0, -200.0, 127.5, 0.333984375, 0.0]
    want = [256, -256, 128, 0, 2, 2, -2, 32767, -32768, 32640, 86, 0]
    got = O.fixed_point(bits(vals))
    assert got.dtype == np.int64
    assert list(got) == want, (list(got), want)


# ---------------------------------------------------------------- dense

def check_dense_vs_sdpa(O):
    rng = _rng(1)
    for Hq, Hkv, N, d in [(2, 1, 70, 16), (4, 2, 33, 64)]:
        q = bits(2 * rng.standard_normal((1, Hq, N, d)))
        k = bits(2 * rng.standard_normal((1, Hkv, N, d)))
        v = bits(rng.standard_normal((1, Hkv, N, d)))
        o, lse = O.dense_causal(q, k, v)
        G = Hq // Hkv
        tq = torch.from_numpy(O.decode_bf16(q))
        tk = torch.from_numpy(O.decode_bf16(k)).repeat_interleave(G, 1)
        tv = torch.from_numpy(O.decode_bf16(v)).repeat_interleave(G, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=True).numpy()
        assert np.abs(o - ref).max() < 1e-12
        # lse against torch.logsumexp over the causal logits
        z = torch.einsum("bhid,bhjd->bhij", tq, tk) / math.sqrt(d)
        z = z.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1),
                          float("-inf"))
        assert np.abs(lse - torch.logsumexp(z, -1).numpy()).max() < 1e-12


def check_dense_closed_forms(O):
    rng = _rng(2)
    N, d = 48, 16
    q = bits(rng.standard_normal((1, 1, N, d)))
    k = np.broadcast_to(bits(rng.standard_normal((1, 1, 1, d))),
                        (1, 1, N, d)).copy()
    v = bits(rng.standard_normal((1, 1, N, d)))
    o, lse = O.dense_causal(q, k, v)
    v64 = O.decode_bf16(v)[0, 0]
    ref = np.cumsum(v64, 0) / np.arange(1, N + 1)[:, None]
    assert np.abs(o[0, 0] - ref).max() < 1e-13
    z = O.decode_bf16(q)[0, 0] @ O.decode_bf16(k)[0, 0, 0] / math.sqrt(d)
    assert np.abs(lse[0, 0] - z - np.log(np.arange(1, N + 1))).max() < 1e-12


# ---------------------------------------------------------------- orders

def _worked_inputs(extra_prefix_keys: bool):
    """N = 256, S = 64, d = 8, one head; answers derived by hand below."""
    N, d = 256, 8
    qf = np.zeros((1, 1, N, d))
    qf[0, 0, :, 0] = 1.0
    m = (np.arange(64) * 37) % 64                 # a permutation of 0..63
    qf[0, 0, 128:192, 1] = (2 * m - 63) / 128.0   # zero-sum, exact in bf16
    kf = np.zeros((1, 1, N, d))
    for j, a in [(5, 2.0), (70, 1.5), (130, 1.0), (200, 0.5)]:
        kf[0, 0, j, 0] = a
    kf[0, 0, 70, 1] = 1.0
    if extra_prefix_keys:
        kf[0, 0, [100, 101, 102], 1] = 1.0
    return bits(qf), bits(kf), m


def check_worked_orders(O):
    """Hand-derived orders.

    fx(q_i) = (256, 4 m_i - 126 in segment 2 else 0, 0...), so the pooled
    query is P = (65536, 0, ...) and v_j = 65536 * 256 * a_j: keys 5, 70,
    130, 200 rank first in that order, all other keys tie at 0 and follow in
    index order. Segment 1: its top tile is all of segment 0, which is also
    its whole prefix, so C_1 = 0 and the order is the identity. Segment 2:
    the top tile of L_2 holds keys 5 and 70, the prefix keys 0..127; the
    second coordinate of C_2 = 128 * top - 64 * prefix is 128 * 256 -
    64 * 256 > 0 with only key 70 carrying it, so queries rank by m
    descending; with keys 100..102 also carrying it (prefix only) it is
    128 * 256 - 64 * 1024 < 0 and queries rank by m ascending. Segment 3's
    queries are identical in the first coordinate and zero elsewhere:
    identity.
    """
    for extra in (False, True):
        q, k, m = _worked_inputs(extra)
        pl = O.plan(q, k, 64)
        hot = [5, 70, 130, 200]
        rest = [j for j in range(256) if j not in hot]
        assert list(pl.pi_k[0, 0]) == hot + rest
        assert list(O.restricted_list(pl, 0, 0, 1)) == [5] + [
            j for j in range(64) if j != 5]
        assert list(O.restricted_list(pl, 0, 0, 2)) == [5, 70] + [
            j for j in range(128) if j not in (5, 70)]
        assert list(O.restricted_list(pl, 0, 0, 3)) == [5, 70, 130] + [
            j for j in range(192) if j not in (5, 70, 130)]
        pq = pl.pi_q[0, 0]
        assert list(pq[:128]) == list(range(128))
        assert list(pq[192:]) == list(range(192, 256))
        local = sorted(range(64), key=(lambda i: m[i]) if extra
                       else (lambda i: -m[i]))
        assert list(pq[128:192]) == [128 + i for i in local]


def check_stripe_score_bruteforce(O):
    """v_j = column sum of the integer logit matrix over all group queries
    (the mean-pooled vertical stripe, up to the factor G N); the orders equal
    ranks obtained by pairwise counting."""
    q, k, _ = _stripe(Hq=2, Hkv=1, N=256, d=16, seed=3)
    pl = O.plan(q, k, 64)
    qx = [O.fixed_point(q[0, h]) for h in range(2)]
    kx = O.fixed_point(k[0, 0])
    col = sum((x @ kx.T).sum(axis=0) for x in qx)
    assert np.array_equal(pl.key_score[0, 0], col)
    v = [int(x) for x in col]
    rank = [sum(1 for j2 in range(256) if (v[j2], -j2) > (v[j], -j))
            for j in range(256)]
    inv = np.empty(256, dtype=np.int64)
    inv[rank] = np.arange(256)
    assert np.array_equal(pl.pi_k[0, 0], inv)
    # query scores: u_i = 64 t S (q_i . mean(top tile) - q_i . mean(prefix))
    S = 64
    for h in range(2):
        for t in (1, 3):
            Lt = O.restricted_list(pl, 0, 0, t)
            top = [Fraction(int(x), 64) for x in kx[Lt[:64]].sum(axis=0)]
            pre = [Fraction(int(x), t * S) for x in kx[:t * S].sum(axis=0)]
            for i in range(t * S, t * S + S, 7):
                qi = [int(x) for x in qx[h][i]]
                u = 64 * t * S * (sum(a * b for a, b in zip(qi, top))
                                  - sum(a * b for a, b in zip(qi, pre)))
                assert u.denominator == 1
                assert int(u) == pl.query_score[0, h, i]


def check_plan_invariants(O):
    q, k, _ = _stripe(Hq=4, Hkv=2, N=1024, d=32, seed=4)
    S = 256
    for flags in (0, O.SA_NO_QPERM, O.SA_NO_KVPERM):
        pl = O.plan(q, k, S, flags=flags)
        for g in range(2):
            pk = pl.pi_k[0, g]
            assert np.array_equal(np.sort(pk), np.arange(1024))
            pos = np.empty(1024, dtype=np.int64)
            pos[pk] = np.arange(1024)
            for t in range(1, 4):
                Lt = O.restricted_list(pl, 0, g, t)
                assert len(Lt) == t * S
                assert np.array_equal(np.sort(Lt), np.arange(t * S))
                assert np.all(np.diff(pos[Lt]) > 0)    # subsequence of pi_K
        for h in range(4):
            pq = pl.pi_q[0, h]
            for t in range(4):
                seg = pq[t * S:(t + 1) * S]
                assert np.array_equal(np.sort(seg), np.arange(t * S,
                                                              (t + 1) * S))
            assert np.array_equal(pq[:S], np.arange(S))   # u = 0 there
        if flags & O.SA_NO_QPERM:
            assert np.array_equal(pl.pi_q[0, 0], np.arange(1024))
        if flags & O.SA_NO_KVPERM:
            assert np.array_equal(pl.pi_k[0, 0], np.arange(1024))


# ---------------------------------------------------------------- S2O

def check_tau0_is_dense(O):
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=64, seed=5)
    od, ld = O.dense_causal(q, k, v)
    for flags in (0, O.SA_NO_QPERM, O.SA_NO_KVPERM,
                  O.SA_NO_QPERM | O.SA_NO_KVPERM, O.SA_SEGMENT_KV,
                  O.SA_SEGMENT_KV | O.SA_NO_QPERM):
        o, lse, *_ = O.s2o_attention(q, k, v, 128, 0.0, flags)
        assert np.abs(o - od).max() < 1e-12
        assert np.abs(lse - ld).max() < 1e-12
    o, *_ = O.s2o_attention(q, k, v, 128, 0.3, O.SA_NO_EARLYSTOP)
    assert np.abs(o - od).max() < 1e-12


def check_kv_order_invariance(O):
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=6)
    od, _ = O.dense_causal(q, k, v)
    perm = _rng(9).permutation(512)[None, None]
    pl = O.plan(q, k, 128, kv_order=perm)
    n_I, _ = O.stop_points(q, k, pl, 0.0)
    o, _ = O.attend(q, k, v, pl, n_I)
    assert np.abs(o - od).max() < 1e-12


def check_single_segment_is_dense(O):
    q, k, v = _stripe(Hq=2, Hkv=1, N=256, d=32, seed=8)
    od, _ = O.dense_causal(q, k, v)
    o, _, _, n_I, _ = O.s2o_attention(q, k, v, 256, 0.5)
    assert np.all(n_I == 0)
    assert np.abs(o - od).max() < 1e-12


def check_bruteforce_restricted(O):
    """Row-by-row attention over an explicitly built key set equals the
    block computation: Sel(i) = own-segment keys j <= i plus the first n_I
    tiles of L_t (brute force, per row, no blocks)."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=384, d=16, seed=10)
    S = 128
    pl = O.plan(q, k, S)
    n_I, _ = O.stop_points(q, k, pl, 0.3)
    full = (np.arange(6) // 2) * 2            # t S / 64 tiles per block
    assert np.any((n_I[0] > 0) & (n_I[0] < full))   # some blocks stop early
    o, lse = O.attend(q, k, v, pl, n_I)
    q64, k64, v64 = (O.decode_bf16(x) for x in (q, k, v))
    for h in range(2):
        block_of_row = np.empty(384, dtype=np.int64)
        block_of_row[pl.pi_q[0, h]] = np.arange(384) // 64
        for i in range(0, 384, 5):
            t = i // S
            sel = [j for j in range(t * S, i + 1)]
            n = int(n_I[0, h, block_of_row[i]])
            if t > 0:
                order = [int(j) for j in pl.pi_k[0, 0] if j < t * S]
                sel += order[:64 * n]
            z = np.array([q64[0, h, i] @ k64[0, 0, j] for j in sel]) / 4.0
            w = np.exp(z - z.max())
            ref = (w[:, None] * v64[0, 0, sel]).sum(0) / w.sum()
            assert np.abs(o[0, h, i] - ref).max() < 1e-12
            assert abs(lse[0, h, i] - (z.max() + np.log(w.sum()))) < 1e-12


def _closed_form_n(tau, D, t, S, r=1.0):
    """First k with r/(D/4096 + r (k + 1)) < tau, for E_diag = (D/64) e^s0
    and E_k = 64 e^s1, r = e^(s1 - s0): k > 1/tau - D/(4096 r) - 1."""
    x = 1.0 / tau - D / (4096.0 * r)
    frac = x - math.floor(x)
    assert 1e-9 < frac < 1 - 1e-9, "case too close to a tie for a pin"
    return min(t * S // 64, max(0, math.floor(x)))


def check_constant_keys_closed_form(O):
    """All keys equal: both orders are the identity (every v_j ties, C_t = 0)
    and every estimate is the same s, so p_k = 64 / (D_I / 64 + 64 (k + 1))
    with D_I = sum_{i in I} (i - t S + 1): n_I = min(t S / 64,
    max(0, floor(1/tau - D_I / 4096))). At exact equality p_k = tau the
    block is still visited (the comparison is strict)."""
    N, d, S = 512, 32, 128
    rng = _rng(12)
    q = bits(rng.standard_normal((1, 1, N, d)))
    v = bits(rng.standard_normal((1, 1, N, d)))
    for kvec in (np.zeros(d), rng.standard_normal(d)):
        k = np.broadcast_to(bits(kvec), (1, 1, N, d)).copy()
        for tau in (0.05, 0.013, 0.125, 0.0625, 1.0, 0.0):
            if tau == 1.0 and kvec.any():
                continue
            pl = O.plan(q, k, S)
            assert np.array_equal(pl.pi_k[0, 0], np.arange(N))
            assert np.array_equal(pl.pi_q[0, 0], np.arange(N))
            n_I, _ = O.stop_points(q, k, pl, tau)
            for I in range(N // 64):
                t = I * 64 // S
                D = sum(i - t * S + 1 for i in range(64 * I, 64 * I + 64))
                want = 0 if t == 0 else (
                    t * S // 64 if tau == 0 else _closed_form_n(tau, D, t, S))
                assert n_I[0, 0, I] == want, (tau, I, n_I[0, 0, I], want)
            # with identical keys the output is the uniform mean over Sel(i)
            if tau == 0.05:
                o, _ = O.attend(q, k, v, pl, n_I)
                v64 = O.decode_bf16(v)[0, 0]
                for i in (130, 300, 511):
                    t = i // S
                    n = int(n_I[0, 0, i // 64])
                    sel = list(range(t * S, i + 1)) + list(range(64 * n))
                    ref = v64[sel].mean(axis=0)
                    assert np.abs(o[0, 0, i] - ref).max() < 1e-12


def check_strict_stop(O):
    """At exact equality p_k = tau the tile is still visited. With zero keys
    every estimate is exp(0) = 1; 64 rows at t S + 63 see all 64 keys of the
    first local block, so E_diag = 64 and p_k = 64 / (64 + 64 (k + 1)) =
    1 / (k + 2): with tau = 1/4, p_2 = tau is visited and k = 3 stops."""
    S, d = 128, 16
    kap = 1.0 / math.sqrt(d)
    local = np.zeros((S // 64, d))
    n, ps = O.block_stop(np.ones(d), np.full(64, S + 63), 1, local,
                         np.zeros((2, d)), S, 0.25, kap)
    assert n == 2 and list(ps) == [0.5, 1 / 3]   # only 2 tiles exist
    n, ps = O.block_stop(np.ones(d), np.full(64, 2 * S + 63), 2, local,
                         np.zeros((4, d)), S, 0.25, kap)
    assert n == 3 and list(ps) == [0.5, 1 / 3, 0.25, 0.2]


def check_two_level_closed_form(O):
    """Segment 0 keys all equal a e_0, segment 1 keys zero (N = 2 S): for a
    block of segment 1 the diagonal estimate is s0 = 0 and every tile's is
    s1 = kappa * qbar_0 * a, so p_k = r / (D_I / 4096 + r (k + 1)) with
    r = exp(s1): the closed form pins kappa, the mean pooling of the query
    block and the 64 keys per row of a sparse tile."""
    N, d, S = 256, 16, 128
    rng = _rng(13)
    qf = rng.standard_normal((1, 1, N, d))
    qf[0, 0, :, 0] += 1.5
    kf = np.zeros((1, 1, N, d))
    kf[0, 0, :S, 0] = 2.0
    q, k = bits(qf), bits(kf)
    pl = O.plan(q, k, S)
    q64 = O.decode_bf16(q)[0, 0]
    assert np.array_equal(pl.pi_q[0, 0, S:], np.arange(S, N))
    for tau in (0.02, 0.04, 0.09):
        n_I, _ = O.stop_points(q, k, pl, tau)
        for I in range(S // 64, N // 64):
            rows = pl.pi_q[0, 0, 64 * I:64 * I + 64]
            D = int((rows - S + 1).sum())
            r = math.exp(q64[rows, 0].mean() * 2.0 / math.sqrt(d))
            assert n_I[0, 0, I] == _closed_form_n(tau, D, 1, S, r), tau


def check_permuted_block_closed_form(O):
    """Two-tile closed form on a permuted query block (N = 2 S, S = 128).

    Segment 0 keys are (1, +1/2, 0...) for the 64 keys of H (odd j) and
    (1, -1/2, 0...) for the others; segment 1 keys are zero. Queries are
    (1, c_i, 0...) with c_i > 0, so P_1 > 0 and the H keys rank first: tile 0
    of L_1 is H (mean (1, 1/2)), tile 1 the rest (mean (1, -1/2)). Then
    C_1 = 128 * top - 64 * prefix = (0, 2^20, 0...), so segment 1's queries
    are ordered by c_i descending. For a block with rows R (that order),
    qbar = (1, mean c over R); the local window has keys 0, so E_diag =
    D / 64 with D = sum_{i in R} (i - S + 1); tile k has E_k = 64 r_k with
    r_0 = exp(kappa (1 + qbar_1 / 2)), r_1 = exp(kappa (1 - qbar_1 / 2)).
    n_I = 0 if r_0 / (D / 4096 + r_0) < tau, else 1 if
    r_1 / (D / 4096 + r_0 + r_1) < tau, else 2.
    """
    N, d, S = 256, 16, 128
    m = (np.arange(128) * 45) % 128               # a permutation of 0..127
    c = np.full(N, 0.5)
    c[S:] = (m + 1) / 64.0                        # exact in bf16
    qf = np.zeros((1, 1, N, d))
    qf[0, 0, :, 0] = 1.0
    qf[0, 0, :, 1] = c
    kf = np.zeros((1, 1, N, d))
    kf[0, 0, :S, 0] = 1.0
    kf[0, 0, :S, 1] = np.where(np.arange(S) % 2 == 1, 0.5, -0.5)
    q, k = bits(qf), bits(kf)
    pl = O.plan(q, k, S)
    order = sorted(range(S, N), key=lambda i: (-c[i], i))
    assert list(pl.pi_q[0, 0, S:]) == order
    kap = 1.0 / math.sqrt(d)
    seen = set()
    for tau in np.linspace(0.05, 0.6, 23):
        n_I, _ = O.stop_points(q, k, pl, float(tau))
        for blk in (0, 1):
            R = np.array(order[64 * blk:64 * blk + 64])
            D = float((R - S + 1).sum())
            qb1 = c[R].mean()
            r0 = math.exp(kap * (1 + qb1 / 2))
            r1 = math.exp(kap * (1 - qb1 / 2))
            if r0 / (D / 4096 + r0) < tau:
                want = 0
            elif r1 / (D / 4096 + r0 + r1) < tau:
                want = 1
            else:
                want = 2
            assert n_I[0, 0, 2 + blk] == want, (tau, blk)
            seen.add((blk, want))
    assert len(seen) >= 5          # the grid exercises every outcome


def check_monotone_tau(O):
    q, k, _ = _stripe(Hq=2, Hkv=1, N=1024, d=32, seed=14)
    pl = O.plan(q, k, 256)
    prev = None
    for tau in (0.0, 0.002, 0.01, 0.03, 0.1, 1.0):
        n_I, _ = O.stop_points(q, k, pl, tau)
        if prev is not None:
            assert np.all(n_I <= prev)
        prev = n_I
    assert np.all(prev == 0)



# ------------------------------------------------- baselines and diagnostics

def check_local_only(O):
    """SA_LOCAL_ONLY visits no tile (also with SA_NO_EARLYSTOP); every row's
    output and lse equal dense causal attention of its own segment taken as
    a sequence of its own (the dense-local-window-only baseline of the S2O
    page's component ablation)."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=9)
    S = 128
    for flags in (O.SA_LOCAL_ONLY, O.SA_LOCAL_ONLY | O.SA_NO_EARLYSTOP):
        pl = O.plan(q, k, S, flags=flags)
        n_I, _ = O.stop_points(q, k, pl, 0.0)
        assert np.all(n_I == 0)
        o, lse = O.attend(q, k, v, pl, n_I)
        for t in range(512 // S):
            sl = slice(t * S, (t + 1) * S)
            od, ld = O.dense_causal(np.ascontiguousarray(q[:, :, sl]),
                                    np.ascontiguousarray(k[:, :, sl]),
                                    np.ascontiguousarray(v[:, :, sl]))
            assert np.abs(o[:, :, sl] - od).max() < 1e-12
            assert np.abs(lse[:, :, sl] - ld).max() < 1e-12


def check_recall(O):
    """Attention recall: 1 when nothing is skipped (tau = 0); otherwise
    exp(lse over Sel(i) - lse over every causal key) with the second from
    torch.logsumexp; within (0, 1] and non-increasing in tau; for
    SA_LOCAL_ONLY the share of the own-segment keys, from explicit index
    sets and torch.logsumexp."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=10)
    N, S, d = 512, 128, 32
    tq = torch.from_numpy(O.decode_bf16(q))
    tk = torch.from_numpy(O.decode_bf16(k)).repeat_interleave(2, 1)
    z = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
    i = torch.arange(N)
    causal = i[None, :] <= i[:, None]
    lse_dense = torch.logsumexp(z.masked_fill(~causal, float("-inf")),
                                -1).numpy()
    pl = O.plan(q, k, S)
    n0, _ = O.stop_points(q, k, pl, 0.0)
    assert np.abs(O.recall(q, k, pl, n0) - 1.0).max() < 1e-12
    prev = None
    for tau in (0.1, 0.3, 0.7):
        n_I, _ = O.stop_points(q, k, pl, tau)
        assert n_I.sum() < n0.sum()
        _, lse_sel = O.attend(q, k, v, pl, n_I)
        r = O.recall(q, k, pl, n_I)
        assert np.abs(r - np.exp(lse_sel - lse_dense)).max() < 1e-10
        assert (r > 0).all() and (r <= 1 + 1e-12).all()
        if prev is not None:
            assert (r <= prev + 1e-12).all()
        prev = r
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.0)
    own = causal & ((i[None, :] // S) == (i[:, None] // S))
    lse_own = torch.logsumexp(z.masked_fill(~own, float("-inf")), -1).numpy()
    assert np.abs(O.recall(q, k, pll, nl) - np.exp(lse_own - lse_dense)
                  ).max() < 1e-10


def check_segment_kv_worked(O):
    """Segment-local key order on a hand-derived example: N = 384, S = 128,
    every query (1, 0, ...), keys with coordinate 0 equal to 1.0 at key 10,
    3.0 at key 100, 2.0 at key 130 and 0 elsewhere, so v_j is proportional
    to that coordinate. Inside segment 0 the order is 100, 10, then the rest
    by index; inside segment 1: 130, then the rest. Tiles (64 keys): A =
    first half of segment 0 (score 4), B = second half (0), C = first half
    of segment 1 (2), D = second half (0). L_1 = A B; L_2 = A C B D (B and
    D tie at 0: smaller tile index first). The global order of the same
    input puts 100, 130, 10 first instead."""
    N, S, d = 384, 128, 8
    qf = np.zeros((1, 1, N, d)); qf[0, 0, :, 0] = 1.0
    kf = np.zeros((1, 1, N, d))
    for j, a in [(10, 1.0), (100, 3.0), (130, 2.0)]:
        kf[0, 0, j, 0] = a
    q, k = bits(qf), bits(kf)
    pl = O.plan(q, k, S, flags=O.SA_SEGMENT_KV)
    seg0 = [100, 10] + [j for j in range(128) if j not in (10, 100)]
    seg1 = [130] + [j for j in range(128, 256) if j != 130]
    seg2 = list(range(256, 384))
    assert pl.pi_k[0, 0].tolist() == seg0 + seg1 + seg2
    A, B, C, D = seg0[:64], seg0[64:], seg1[:64], seg1[64:]
    assert O.restricted_list(pl, 0, 0, 1).tolist() == A + B
    assert O.restricted_list(pl, 0, 0, 2).tolist() == A + C + B + D
    g = O.plan(q, k, S)
    assert g.pi_k[0, 0, :3].tolist() == [100, 130, 10]


def check_segment_kv_invariants(O):
    """On stripe inputs: pi_K permutes each segment and orders it by v
    descending (ties by index); every L_t is a concatenation of 64-key
    chunks of pi_K[0 : t S] (each chunk once) with non-increasing sums of
    v; SA_NO_KVPERM still gives the identity order."""
    q, k, v = _stripe(Hq=4, Hkv=2, N=1024, d=32, seed=12)
    S = 256
    pl = O.plan(q, k, S, flags=O.SA_SEGMENT_KV)
    for g in range(2):
        pk, vs = pl.pi_k[0, g], pl.key_score[0, g]
        for u in range(1024 // S):
            seg = pk[u * S:(u + 1) * S]
            assert sorted(seg.tolist()) == list(range(u * S, (u + 1) * S))
            for a_, b_ in zip(seg[:-1], seg[1:]):
                assert vs[a_] > vs[b_] or (vs[a_] == vs[b_] and a_ < b_)
        chunks = {tuple(pk[i:i + 64].tolist()): i // 64
                  for i in range(0, 1024, 64)}
        for t in range(1, 1024 // S):
            Lt = O.restricted_list(pl, 0, g, t)
            tiles = [tuple(Lt[i:i + 64].tolist()) for i in range(0, len(Lt), 64)]
            ids = [chunks[x] for x in tiles]
            assert sorted(ids) == list(range(t * S // 64))
            sums = [int(vs[list(x)].sum()) for x in tiles]
            for i in range(len(sums) - 1):
                assert sums[i] > sums[i + 1] or (
                    sums[i] == sums[i + 1] and ids[i] < ids[i + 1])
    pid = O.plan(q, k, S, flags=O.SA_SEGMENT_KV | O.SA_NO_KVPERM)
    assert np.array_equal(pid.pi_k[0, 0], np.arange(1024))


def check_budget(O):
    """Fixed tile budget: n_I = min(K, t S / 64) in segment t (closed
    form); K = 0 gives the dense-local-window-only outputs; a budget of
    every tile gives dense attention; matched visits differ from the tau
    stop's per-block counts (the budget is the same for every block)."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=13)
    S = 128
    pl = O.plan(q, k, S)
    for K in (0, 1, 3, 100):
        n_I, _ = O.stop_points(q, k, pl, 0.7, budget=K)
        for I in range(512 // 64):
            t = I * 64 // S
            assert (n_I[0, :, I] == min(K, t * S // 64)).all()
    n0, _ = O.stop_points(q, k, pl, 0.3, budget=0)
    o0, l0 = O.attend(q, k, v, pl, n0)
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.3)
    ol, ll = O.attend(q, k, v, pll, nl)
    assert np.abs(o0 - ol).max() < 1e-12 and np.abs(l0 - ll).max() < 1e-12
    nall, _ = O.stop_points(q, k, pl, 0.9, budget=512 // 64)
    oall, _ = O.attend(q, k, v, pl, nall)
    od, _ = O.dense_causal(q, k, v)
    assert np.abs(oall - od).max() < 1e-12
    nb, _ = O.stop_points(q, k, pll, 0.0, budget=5)
    assert (nb == 0).all()  # SA_LOCAL_ONLY takes precedence


def check_exact_max(O):
    """Exact per-block maximum test: tile maxima by brute force (library
    einsum over the explicit tile keys), selection = maxima >= theta;
    theta = -inf gives dense attention, theta = +inf the dense local window
    only; the selected set shrinks as theta grows."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=14)
    S, d = 128, 32
    pl = O.plan(q, k, S)
    tq = torch.from_numpy(O.decode_bf16(q))
    tk = torch.from_numpy(O.decode_bf16(k))
    _, _, mx = O.exact_max_selection(q, k, pl, 0.0)
    for (b, h, I), m in mx.items():
        t = I * 64 // S
        if t == 0:
            continue
        rows = torch.from_numpy(pl.pi_q[b, h, I * 64:(I + 1) * 64])
        tiles = O.restricted_list(pl, b, 0, t).reshape(-1, 64)
        for c in range(tiles.shape[0]):
            keys = torch.from_numpy(tiles[c])
            z = torch.einsum("id,jd->ij", tq[b, h][rows], tk[b, 0][keys])
            assert abs(float(z.amax()) / math.sqrt(d) - m[c]) < 1e-12
    vals = np.concatenate([m for m in mx.values() if len(m)])
    theta = float(np.sort(vals)[len(vals) // 2])  # an attained maximum
    n_I, masks, _ = O.exact_max_selection(q, k, pl, theta)
    for key, m in mx.items():
        assert np.array_equal(masks[key], m >= theta)
        assert n_I[key] == int((m >= theta).sum())
    od, _ = O.dense_causal(q, k, v)
    n_all, m_all, _ = O.exact_max_selection(q, k, pl, -np.inf)
    o_all, _ = O.attend(q, k, v, pl, n_all, tile_mask=m_all)
    assert np.abs(o_all - od).max() < 1e-12
    n_no, m_no, _ = O.exact_max_selection(q, k, pl, np.inf)
    o_no, _ = O.attend(q, k, v, pl, n_no, tile_mask=m_no)
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.0)
    ol, _ = O.attend(q, k, v, pll, nl)
    assert np.abs(o_no - ol).max() < 1e-12
    hi, _, _ = O.exact_max_selection(q, k, pl, theta + 0.5)
    assert (hi <= n_I).all() and hi.sum() < n_I.sum()


# ------------------------------------------------------------------ metrics

def check_selected_counts_bruteforce(O):
    """|Sel(i)| of every row against an explicitly built key set (own-segment
    keys j <= i plus the keys of the first n_I tiles of L_t, collected row
    by row with the block of each row looked up in pi_Q), on a plan whose
    query order is not the identity and with stop points that differ from
    block to block."""
    q, k, _ = _stripe(Hq=2, Hkv=1, N=384, d=16, seed=10)
    S = 128
    pl = O.plan(q, k, S)
    n_I, _ = O.stop_points(q, k, pl, 0.3)
    assert len(set(n_I[0, :, 2:].ravel().tolist())) > 1
    assert not np.array_equal(pl.pi_q[0, 0], np.arange(384))
    cnt = O.selected_counts(pl, n_I)
    for h in range(2):
        block_of_row = np.empty(384, dtype=np.int64)
        block_of_row[pl.pi_q[0, h]] = np.arange(384) // 64
        for i in range(384):
            t = i // S
            sel = set(range(t * S, i + 1))
            n = int(n_I[0, h, block_of_row[i]])
            if t > 0:
                order = [int(j) for j in pl.pi_k[0, 0] if j < t * S]
                sel |= set(order[:64 * n])
            assert cnt[0, h, i] == len(sel), (h, i)


def check_metrics_closed_forms(O):
    """Pair sparsity (S2O page, Key points: the share of causal query-key
    pairs skipped) in closed forms: 0 when nothing is skipped (tau = 0, or a
    single segment at any tau); 1 - T S (S + 1) / (N (N + 1)) for the dense
    local window only (each row sees the keys of its own segment up to
    itself). Tile density: exactly 1 at tau = 0 with the identity query
    order (block i of a segment touches local blocks 0..i, and all t S / 64
    tiles of L_t); with constant keys (identity orders) it is
    (sum of (i + 1) over the blocks + sum of n_I) over nb (nb + 1) / 2 with
    n_I from the constant-key closed form. MSE: the mean of the squared
    differences, against torch's mse_loss."""
    q, k, v = _stripe(B=2, Hq=2, Hkv=1, N=512, d=32, seed=15)
    N, S = 512, 128
    T, nb = N // S, N // 64
    for flags in (0, O.SA_NO_QPERM):
        pl = O.plan(q, k, S, flags=flags)
        n0, _ = O.stop_points(q, k, pl, 0.0)
        m = O.metrics(pl, n0)
        assert m["pair_sparsity"] == 0.0
        if flags:
            assert m["tile_density"] == 1.0
        else:
            assert m["tile_density"] > 1.0     # permuted blocks spread out
    one = O.plan(q, k, N)
    n1, _ = O.stop_points(q, k, one, 0.4)
    assert O.metrics(one, n1)["pair_sparsity"] == 0.0
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.0)
    want = 1.0 - T * S * (S + 1) / (N * (N + 1))
    assert abs(O.metrics(pll, nl)["pair_sparsity"] - want) < 1e-15
    # constant keys: identity orders, n_I in closed form
    rng = _rng(16)
    d = 32
    qc = bits(rng.standard_normal((1, 1, N, d)))
    kc = np.broadcast_to(bits(rng.standard_normal(d)), (1, 1, N, d)).copy()
    plc = O.plan(qc, kc, S)
    tau = 0.05
    nc, _ = O.stop_points(qc, kc, plc, tau)
    visited = 0
    pairs = 0
    for I in range(nb):
        t = I * 64 // S
        i_loc = (I * 64 - t * S) // 64
        D = sum(i - t * S + 1 for i in range(64 * I, 64 * I + 64))
        n = 0 if t == 0 else _closed_form_n(tau, D, t, S)
        visited += i_loc + 1 + n
        pairs += D + 4096 * n
    mc = O.metrics(plc, nc)
    assert abs(mc["tile_density"] - visited / (nb * (nb + 1) / 2)) < 1e-15
    assert abs(mc["pair_sparsity"] - (1 - pairs / (N * (N + 1) / 2))) < 1e-15
    assert mc["visited_sparse_tiles"] == int(nc.sum())
    # a hand-made query order of one segment of 128 rows: block 0 holds
    # rows 1..64 (row 64 sees key 64, the first key of local block 1: one
    # visible pair there), block 1 rows 0 and 65..127; each block touches
    # both local blocks, so 4 of the nb (nb + 1) / 2 = 3 causal tiles
    one2 = O.plan(q[:, :, :128], k[:, :, :128], 128)
    pq = np.concatenate([np.arange(1, 65), [0], np.arange(65, 128)])
    hand = dataclasses.replace(one2, pi_q=np.broadcast_to(
        pq, one2.pi_q.shape).copy())
    mh = O.metrics(hand, np.zeros((2, 2, 2), dtype=np.int64))
    assert mh["tile_density"] == 4 / 3 and mh["pair_sparsity"] == 0.0
    # MSE
    o = rng.standard_normal((2, 2, 8, 4))
    od = rng.standard_normal((2, 2, 8, 4))
    mse = O.metrics(pl, n0, o, od)["mse"]
    ref = torch.nn.functional.mse_loss(torch.from_numpy(o),
                                       torch.from_numpy(od)).item()
    assert abs(mse - ref) < 1e-15


# ------------------------------------------------- centroid Top-K selection

def check_topk_bruteforce(O):
    """Per-block Top-K from mean-pooled centroids: each tile's score is the
    sum of the block's 64 x 64 matrix of integer logits fx(q_i) . fx(k_j)
    over its rows and the tile's keys (by bilinearity the pooled product);
    the selection holds the tiles whose rank, counted pairwise on (score,
    -position), is below K; n_I counts them."""
    q, k, _ = _stripe(Hq=2, Hkv=1, N=512, d=16, seed=17)
    S = 128
    pl = O.plan(q, k, S)
    qx = [O.fixed_point(q[0, h]) for h in range(2)]
    kx = O.fixed_point(k[0, 0])
    for K in (1, 3, 5):
        n_I, masks, scores = O.topk_selection(q, k, pl, K)
        for h in range(2):
            for I in range(512 // 64):
                t = I * 64 // S
                ntl = t * S // 64
                rows = pl.pi_q[0, h, 64 * I:64 * I + 64]
                if t == 0:
                    assert n_I[0, h, I] == 0 and not masks[(0, h, I)].any()
                    continue
                tiles = O.restricted_list(pl, 0, 0, t).reshape(-1, 64)
                r = [int((qx[h][rows] @ kx[tiles[c]].T).sum())
                     for c in range(ntl)]
                assert [int(x) for x in scores[(0, h, I)]] == r
                rank = [sum(1 for c2 in range(ntl)
                            if (r[c2], -c2) > (r[c], -c)) for c in range(ntl)]
                want = [rk < K for rk in rank]
                assert masks[(0, h, I)].tolist() == want, (K, h, I)
                assert n_I[0, h, I] == min(K, ntl)


def check_topk_worked(O):
    """Hand-derived selection (N = 384, S = 128, d = 8). Segment 0's queries
    are e1 (coordinate 0 = 1), segment 1's rows 128..191 e2 and 192..255
    e1, segment 2's rows zero; keys 0..63 are e1, keys 64..127 e2, the rest
    zero. The pooled query is 256 (192 e1 + 64 e2), so the e1 keys rank
    first: L_1 = [e1 tile, e2 tile], L_2 = [e1, e2, keys 128..191, keys
    192..255]. C_1 = 2^20 (e1 - e2), so segment 1's order puts the e1
    queries first: block 2 = rows 192..255, block 3 = rows 128..191.
    K = 1: block 2 takes the e1 tile, block 3 the e2 tile (a fixed budget
    would give both the e1 tile); segment 2's zero queries score every tile
    0, so ties go to the first positions: K = 1 -> tile 0, K = 3 -> tiles
    0..2; K = 9 -> every tile."""
    N, d, S = 384, 8, 128
    qf = np.zeros((1, 1, N, d))
    qf[0, 0, :128, 0] = 1.0
    qf[0, 0, 128:192, 1] = 1.0
    qf[0, 0, 192:256, 0] = 1.0
    kf = np.zeros((1, 1, N, d))
    kf[0, 0, :64, 0] = 1.0
    kf[0, 0, 64:128, 1] = 1.0
    q, k = bits(qf), bits(kf)
    pl = O.plan(q, k, S)
    assert list(pl.pi_q[0, 0, 128:256]) == list(range(192, 256)) + list(
        range(128, 192))
    want = {1: {2: [1, 0], 3: [0, 1], 4: [1, 0, 0, 0], 5: [1, 0, 0, 0]},
            3: {2: [1, 1], 3: [1, 1], 4: [1, 1, 1, 0], 5: [1, 1, 1, 0]},
            9: {2: [1, 1], 3: [1, 1], 4: [1, 1, 1, 1], 5: [1, 1, 1, 1]}}
    for K, per_block in want.items():
        n_I, masks, _ = O.topk_selection(q, k, pl, K)
        for I, m in per_block.items():
            assert masks[(0, 0, I)].astype(int).tolist() == m, (K, I)
            assert n_I[0, 0, I] == sum(m)
        assert n_I[0, 0, 0] == n_I[0, 0, 1] == 0


def check_topk_closed_forms(O):
    """K = 0 attends the dense local window only (the SA_LOCAL_ONLY
    outputs); K at least the number of tiles attends everything (dense
    attention); SA_LOCAL_ONLY attends to no tile whatever K."""
    q, k, v = _stripe(Hq=2, Hkv=1, N=512, d=32, seed=18)
    S = 128
    pl = O.plan(q, k, S)
    n0, m0, _ = O.topk_selection(q, k, pl, 0)
    o0, l0 = O.attend(q, k, v, pl, n0, tile_mask=m0)
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.0)
    ol, ll = O.attend(q, k, v, pll, nl)
    assert (n0 == 0).all()
    assert np.abs(o0 - ol).max() < 1e-12 and np.abs(l0 - ll).max() < 1e-12
    na, ma, _ = O.topk_selection(q, k, pl, 512 // 64)
    oa, la = O.attend(q, k, v, pl, na, tile_mask=ma)
    od, ld = O.dense_causal(q, k, v)
    assert np.abs(oa - od).max() < 1e-12 and np.abs(la - ld).max() < 1e-12
    nL, mL, _ = O.topk_selection(q, k, pll, 3)
    assert (nL == 0).all() and not any(m.any() for m in mL.values())


ALL_CHECKS = [
    check_fixed_point, check_dense_vs_sdpa, check_dense_closed_forms,
    check_worked_orders, check_stripe_score_bruteforce, check_plan_invariants,
    check_tau0_is_dense, check_kv_order_invariance,
    check_single_segment_is_dense, check_bruteforce_restricted,
    check_constant_keys_closed_form, check_strict_stop,
    check_two_level_closed_form, check_permuted_block_closed_form,
    check_monotone_tau, check_local_only, check_recall,
    check_segment_kv_worked, check_segment_kv_invariants, check_budget,
    check_exact_max, check_selected_counts_bruteforce,
    check_metrics_closed_forms, check_topk_bruteforce, check_topk_worked,
    check_topk_closed_forms,
]
