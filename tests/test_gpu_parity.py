"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Indices and integer scores must match bit for bit; stop points must match
except on documented near-tau ties; outputs must be within 2e-2 max-abs and
1e-4 MSE of the float64 oracle evaluated on the same stop points.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import (StripeSpec, bf16_bits_to_float32, get_config,
                       make_stripe_inputs, round_to_bf16_bits)
from tests.gpu_helpers import (LSE_TOL, assert_outputs_close, assert_plan_equal,
                               run_gpu, say, stop_mismatches)

pytestmark = pytest.mark.gpu


def _spec(B, Hq, Hkv, N, seed, n_vert=16, n_horiz=8, window=64):
    return StripeSpec(B, Hq, Hkv, N, 128, n_vert=n_vert, n_horiz=n_horiz,
                      window=window, seed=seed)


CASES = [
    # name, spec, segment, taus, flags
    ("tiny_n2048_s512", get_config(1).spec, 512, (0.005, 0.05, 0.2), 0),
    ("gqa_b2_h4_kv2_n1024", _spec(2, 4, 2, 1024, 21), 256, (0.0, 0.02, 0.1),
     0),
    ("ragged_n640_s128", _spec(1, 2, 1, 640, 22), 128, (0.05, 0.3), 0),
    ("s64_one_block_per_segment", _spec(1, 2, 2, 768, 23), 64, (0.1, 0.4), 0),
    # 4 of the 8 waves of each workgroup hold no query rows and run ahead
    ("s64_g2_idle_waves", _spec(1, 2, 1, 768, 23), 64, (0.1, 0.4), 0),
    ("g8_h8_kv1_n512", _spec(1, 8, 1, 512, 24), 128, (0.03,), 0),
    ("single_segment_n256", _spec(1, 2, 1, 256, 25), 256, (0.5,), 0),
    ("single_block_n64", _spec(1, 1, 1, 64, 26, n_vert=2, n_horiz=1,
                               window=16), 64, (0.1,), 0),
    ("no_qperm", _spec(1, 4, 1, 1024, 27), 256, (0.05,), O.SA_NO_QPERM),
    ("no_kvperm", _spec(1, 4, 1, 1024, 28), 256, (0.05,), O.SA_NO_KVPERM),
    ("no_earlystop", _spec(1, 2, 1, 1024, 29), 256, (0.2,), O.SA_NO_EARLYSTOP),
    ("local_only", _spec(1, 4, 2, 1024, 32), 256, (0.0, 0.05),
     O.SA_LOCAL_ONLY),
    ("local_only_no_earlystop", _spec(1, 2, 1, 640, 33), 128, (0.0,),
     O.SA_LOCAL_ONLY | O.SA_NO_EARLYSTOP),
    ("segment_kv", _spec(1, 4, 2, 1024, 35), 256, (0.0, 0.05, 0.2),
     O.SA_SEGMENT_KV),
    ("segment_kv_s64", _spec(1, 2, 1, 768, 36), 64, (0.1, 0.4),
     O.SA_SEGMENT_KV),
    ("segment_kv_no_qperm", _spec(1, 2, 1, 1024, 37), 256, (0.05,),
     O.SA_SEGMENT_KV | O.SA_NO_QPERM),
    ("segment_kv_t64_n16384", _spec(1, 1, 1, 16384, 38, n_vert=32,
                                    window=128), 256, (0.05,),
     O.SA_SEGMENT_KV),
    ("s4096_merge_sort_n8192", _spec(1, 2, 1, 8192, 30, n_vert=64,
                                     window=128), 4096, (0.02,), 0),
    # pi_K: three sort chunks, so the merge passes meet a pair with no second
    # run and then a short second run; pi_Q: segments of 6144 = 4096 + 2048
    # (a padded chunk and a merge pass over the segment)
    ("ragged_merges_n12288_s6144", _spec(1, 2, 1, 12288, 40, n_vert=64,
                                         window=128), 6144, (0.05,), 0),
    # 64 query heads per KV head: 2048 query blocks per (KV head, segment),
    # more than the sparse pass orders by stop point (it takes them in order)
    ("g64_blocks_in_order_n4096", _spec(1, 64, 1, 4096, 42), 2048, (0.05,),
     0),
    # 4 query heads x 64 blocks per segment: the stop scan splits a segment's
    # 256 blocks over two workgroups and its 64 local blocks over two chunks
    ("g4_s4096_two_scan_chunks", _spec(1, 4, 1, 8192, 39, n_vert=64,
                                       window=128), 4096, (0.02, 0.1), 0),
    # the local pass with two blocks per workgroup (4 query heads per KV
    # head): pairs (3, 0) and (2, 1), whose first blocks end after an even
    # and an odd number of steps, with and without the sparse pass after it
    ("local_pairs_g4_s256", _spec(1, 8, 2, 1024, 60), 256, (0.02, 0.1), 0),
    ("local_only_pairs_g4_s256", _spec(1, 8, 2, 1024, 61), 256, (0.0,),
     O.SA_LOCAL_ONLY),
    # one pair per segment: (1, 0)
    ("local_pairs_g4_s128", _spec(1, 4, 1, 512, 62), 128, (0.05,), 0),
]


def _check_case(q, k, v, S, tau, flags):
    pl = O.plan(q, k, S, flags=flags)
    n_orc, traces = O.stop_points(q, k, pl, tau)
    g = run_gpu(q, k, v, S, tau, flags)
    assert_plan_equal(g, pl)
    ties = stop_mismatches(g["n_I"], n_orc, traces,
                           0.0 if flags & O.SA_NO_EARLYSTOP else tau)
    n_use = n_orc.copy()
    for b, h, I in ties:
        n_use[b, h, I] = g["n_I"][b, h, I]
    o_ref, lse_ref = O.attend(q, k, v, pl, n_use)
    err, mse = assert_outputs_close(g["o"], o_ref, g["lse"], lse_ref)
    return err, mse, len(ties), g, pl, n_orc


@pytest.mark.parametrize("name,spec,S,taus,flags", CASES,
                         ids=[c[0] for c in CASES])
def test_parity_small(name, spec, S, taus, flags):
    q, k, v = make_stripe_inputs(spec)
    for tau in taus:
        say(f"[parity] {name} tau={tau} flags={flags}")
        err, mse, nties, g, pl, n_orc = _check_case(q, k, v, S, tau, flags)
        say(f"   max_abs={err:.3g} mse={mse:.3g} ties={nties} "
            f"mean_n_I={g['n_I'].mean():.2f}")


C2 = 1.4426950408889634 / np.sqrt(128.0)  # kappa log2(e), d = 128


def _reference_margins(qf, kf, S):
    """Per (head, row): |q| max_j |k_j| kappa log2(e) (with the kernel's 2^-10
    margin) minus the row's largest logit over its segment's first 64 keys,
    and the rise of the row's largest logit over all visible keys above that
    first one (log2 units, float64)."""
    B, Hq, N, d = qf.shape
    G = Hq // kf.shape[1]
    margin = np.zeros((Hq, N))
    rise = np.zeros((Hq, N))
    for h in range(Hq):
        K, Q = kf[0, h // G], qf[0, h]
        L = (Q @ K.T) * C2
        kmax = np.sqrt((K * K).sum(-1).max())
        qn = np.sqrt((Q * Q).sum(-1))
        for i in range(N):
            s0 = (i // S) * S
            m0 = L[i, s0:min(s0 + 64, i + 1)].max()
            margin[h, i] = qn[i] * kmax * C2 * (1 + 1 / 1024) - m0
            rise[h, i] = L[i, :i + 1].max() - m0
    return margin, rise


def test_reference_paths():
    """Both references of the online softmax against the oracle. Head 0:
    four late keys pulled towards the mean query, so that some rows' logits
    rise more than 8 log2 units above the first local tile's maximum (the
    rescale of the bounded path runs) while every row stays provably
    bounded. Head 1: queries and keys times 4 (exact in bf16), so that its
    rows are not provably bounded and its workgroups run with the row
    maximum of every tile. One query block per workgroup head (G = 1), so
    both kinds of workgroup run in the same launch."""
    spec = _spec(1, 2, 2, 1024, 41)
    S = 256
    q, k, v = make_stripe_inputs(spec)
    qf = bf16_bits_to_float32(q).astype(np.float64)
    kf = bf16_bits_to_float32(k).astype(np.float64)
    qbar = qf[0, 0].mean(0)
    qbar /= np.linalg.norm(qbar)
    for j in (200, 500, 777, 900):
        kf[0, 0, j] += 10.0 * qbar * np.sqrt(128.0) / 4
    qf[0, 1] *= 4.0
    kf[0, 1] *= 4.0
    q = round_to_bf16_bits(qf.astype(np.float32))
    k = round_to_bf16_bits(kf.astype(np.float32))
    qf = bf16_bits_to_float32(q).astype(np.float64)
    kf = bf16_bits_to_float32(k).astype(np.float64)
    margin, rise = _reference_margins(qf, kf, S)
    assert margin[0].max() < 120.0 and (rise[0] > 8.0).sum() >= 10
    assert margin[1].min() > 120.0
    for tau in (0.0, 0.05):
        say(f"[reference paths] tau={tau}")
        err, mse, nties, g, pl, n_orc = _check_case(q, k, v, S, tau, 0)
        say(f"   max_abs={err:.3g} mse={mse:.3g} ties={nties}")
    od, ld = O.dense_causal(q, k, v)
    g = run_gpu(q, k, v, S, 0.0)
    assert_outputs_close(g["o"], od, g["lse"], ld)


def test_forward_matches_plan_then_prefill():
    """sparse_attn_forward (local windows on a second stream while the
    planner runs) returns what plan + prefill return, bit for bit, and so
    does its one-stream form; the plan it returns serves a further prefill
    at another tau."""
    import torch
    import permuted_block_sparse_amd as pbs
    from tests.gpu_helpers import to_device
    side = torch.cuda.Stream()
    # the local pass with pairs of blocks (4 query heads per KV head, an
    # even number of blocks per segment), one block per workgroup (2 heads
    # per KV head; 3 heads and 5 blocks per segment), a batch of two with
    # the segment-local KV order
    shapes = [(_spec(1, 4, 1, 4096, 43, n_vert=32, window=128), 512, 0.05, 0),
              (_spec(1, 4, 2, 2048, 44), 256, 0.02, 0),
              (_spec(1, 3, 1, 1600, 45), 320, 0.05, 0),
              (_spec(2, 8, 2, 1024, 46), 256, 0.1, O.SA_SEGMENT_KV)]
    for spec, S, tau, flags in shapes:
        q, k, v = make_stripe_inputs(spec)
        tq, tk, tv = to_device(q), to_device(k), to_device(v)
        pl = pbs.plan(tq, tk, S, tau, flags=flags)
        o_ref, l_ref = pbs.prefill(pl, tq, tk, tv, return_lse=True)
        torch.cuda.synchronize()
        for name, ss in (("side stream", side), ("one stream", None)):
            say(f"[forward] B={spec.batch} Hq={spec.heads_q} "
                f"Hkv={spec.heads_kv} N={spec.seq_len} S={S} {name}")
            pf, o, l = pbs.forward(tq, tk, tv, S, tau, flags=flags,
                                   return_lse=True, side_stream=ss)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
            assert torch.equal(l, l_ref)
            for ex in ("pi_k", "pi_q", "restricted_lists", "n_I"):
                assert np.array_equal(getattr(pf, ex)(),
                                      getattr(pl, ex)()), ex
    pf.set_tau(0.2)
    pl.set_tau(0.2)
    o2 = pbs.prefill(pf, tq, tk, tv)
    o2_ref = pbs.prefill(pl, tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o2_ref.view(torch.int16))


def test_tau0_is_dense_and_kv_order_invariant():
    spec = _spec(1, 4, 2, 1024, 31)
    q, k, v = make_stripe_inputs(spec)
    od, ld = O.dense_causal(q, k, v)
    say("[parity] tau=0 vs dense")
    g = run_gpu(q, k, v, 256, 0.0)
    assert_outputs_close(g["o"], od, g["lse"], ld)
    perm = np.stack([np.random.default_rng(5 + i).permutation(1024)
                     for i in range(2)])[None]
    say("[parity] tau=0 with an injected KV order vs dense")
    g2 = run_gpu(q, k, v, 256, 0.0, kv_order=perm)
    assert np.array_equal(g2["pi_k"], perm)
    pl = O.plan(q, k, 256, kv_order=perm)
    assert np.array_equal(g2["L"], pl.L)
    assert np.array_equal(g2["pi_q"], pl.pi_q)
    assert_outputs_close(g2["o"], od, g2["lse"], ld)


def test_recall_from_lse():
    """Attention recall from two GPU runs, exp(lse at tau - lse at tau = 0),
    against the oracle's brute-force recall (the share of each row's dense
    causal attention mass on its selected set); also for the dense local
    window only."""
    spec = _spec(1, 4, 2, 1024, 34)
    q, k, v = make_stripe_inputs(spec)
    S = 256
    say("[recall] tau = 0 reference run")
    g0 = run_gpu(q, k, v, S, 0.0)
    for tau, flags in ((0.05, 0), (0.3, 0), (0.0, O.SA_LOCAL_ONLY)):
        say(f"[recall] tau={tau} flags={flags}")
        g = run_gpu(q, k, v, S, tau, flags)
        pl = O.plan(q, k, S, flags=flags)
        n_I = g["n_I"].astype(np.int64)  # recall of the GPU's own selection
        r_ref = O.recall(q, k, pl, n_I)
        r_gpu = np.exp(g["lse"] - g0["lse"])
        assert np.abs(r_gpu - r_ref).max() <= 5e-3, np.abs(r_gpu - r_ref).max()
        if flags == 0 and tau > 0.1:
            assert r_ref.mean() < 1.0 - 1e-6  # something was skipped


def test_segment_kv_worked_example():
    """The hand-derived segment-local example on the GPU plan (head
    dimension zero-padded to 128): N = 384, S = 128, every query
    (1, 0, ...), key coordinate 0 = 1.0 at key 10, 3.0 at key 100, 2.0 at
    key 130. Segment orders 100, 10, rest / 130, rest; tiles A, B (segment
    0, scores 4 and 0), C, D (segment 1, scores 2 and 0); L_1 = A B and
    L_2 = A C B D. Injecting a KV order into such a plan is refused."""
    import permuted_block_sparse_amd as pbs
    N, S = 384, 128
    qf = np.zeros((1, 1, N, 128), np.float32)
    qf[0, 0, :, 0] = 1.0
    kf = np.zeros((1, 1, N, 128), np.float32)
    for j, a in [(10, 1.0), (100, 3.0), (130, 2.0)]:
        kf[0, 0, j, 0] = a
    q, k = round_to_bf16_bits(qf), round_to_bf16_bits(kf)
    say("[segment_kv] worked example")
    g = run_gpu(q, k, np.zeros_like(q), S, 0.0, O.SA_SEGMENT_KV)
    seg0 = [100, 10] + [j for j in range(128) if j not in (10, 100)]
    seg1 = [130] + [j for j in range(128, 256) if j != 130]
    assert g["pi_k"][0, 0].tolist() == seg0 + seg1 + list(range(256, 384))
    A, B, C, D = seg0[:64], seg0[64:], seg1[:64], seg1[64:]
    L = g["L"][0, 0]
    assert L[:128].tolist() == A + B
    assert L[128:384].tolist() == A + C + B + D
    with pytest.raises(pbs.SparseAttnError):
        g["plan"].set_kv_order(torch_arange_order(N))


def torch_arange_order(N):
    import torch
    return torch.arange(N, dtype=torch.int32, device="cuda:0").view(1, 1, N)


def test_budget_parity():
    """Fixed tile budget instead of the tau stop: n_I = min(K, t S / 64)
    exactly, outputs against the oracle on those stop points; a negative
    budget restores the tau stop."""
    spec = _spec(1, 4, 2, 1024, 39)
    q, k, v = make_stripe_inputs(spec)
    S = 256
    pl = O.plan(q, k, S)
    for K in (0, 2, 7):
        say(f"[budget] K={K}")
        g = run_gpu(q, k, v, S, 0.05, budget=K)
        n_ref, _ = O.stop_points(q, k, pl, 0.05, budget=K)
        assert np.array_equal(g["n_I"], n_ref)
        o_ref, l_ref = O.attend(q, k, v, pl, n_ref)
        assert_outputs_close(g["o"], o_ref, g["lse"], l_ref)
    say("[budget] back to the tau stop")
    g = run_gpu(q, k, v, S, 0.05, budget=-1)
    n_tau, traces = O.stop_points(q, k, pl, 0.05)
    assert not stop_mismatches(g["n_I"], n_tau, traces, 0.05)


def test_exact_max_parity():
    """Exact per-block maximum test: attended-tile counts equal the
    oracle's and outputs match the oracle on its tile masks, at thresholds
    placed in gaps of at least 2e-3 between the oracle's tile maxima (fp32
    against float64 maxima cannot disagree there); theta = -inf gives dense
    attention, +inf the local window only, NaN restores the tau stop."""
    spec = _spec(1, 4, 2, 1024, 40)
    q, k, v = make_stripe_inputs(spec)
    S = 256
    pl = O.plan(q, k, S)
    _, _, mx = O.exact_max_selection(q, k, pl, 0.0)
    vals = np.sort(np.concatenate([m for m in mx.values() if len(m)]))
    gaps = np.flatnonzero(np.diff(vals) >= 2e-3)
    for frac in (0.3, 0.7):
        i = gaps[np.searchsorted(gaps, int(frac * len(vals)))]
        theta = float((vals[i] + vals[i + 1]) / 2)
        say(f"[exact] theta={theta:.4f}")
        g = run_gpu(q, k, v, S, 0.05, max_theta=theta)
        n_ref, masks, _ = O.exact_max_selection(q, k, pl, theta)
        assert np.array_equal(g["n_I"], n_ref)
        o_ref, l_ref = O.attend(q, k, v, pl, n_ref, tile_mask=masks)
        assert_outputs_close(g["o"], o_ref, g["lse"], l_ref)
    od, ld = O.dense_causal(q, k, v)
    say("[exact] theta=-inf")
    g = run_gpu(q, k, v, S, 0.05, max_theta=-np.inf)
    assert_outputs_close(g["o"], od, g["lse"], ld)
    say("[exact] theta=+inf")
    g = run_gpu(q, k, v, S, 0.05, max_theta=np.inf)
    assert (g["n_I"] == 0).all()
    pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
    nl, _ = O.stop_points(q, k, pll, 0.0)
    ol, ll = O.attend(q, k, v, pll, nl)
    assert_outputs_close(g["o"], ol, g["lse"], ll)
    say("[exact] theta=NaN (tau stop)")
    g = run_gpu(q, k, v, S, 0.05, max_theta=float("nan"))
    n_tau, traces = O.stop_points(q, k, pl, 0.05)
    assert not stop_mismatches(g["n_I"], n_tau, traces, 0.05)


def test_deterministic():
    spec = _spec(1, 4, 1, 2048, 32)
    q, k, v = make_stripe_inputs(spec)
    say("[parity] determinism")
    a = run_gpu(q, k, v, 512, 0.02)
    b = run_gpu(q, k, v, 512, 0.02)
    for key in ("o", "lse", "pi_k", "pi_q", "L", "n_I"):
        assert np.array_equal(a[key], b[key]), key


def test_causal_values_and_later_segments():
    spec = _spec(1, 2, 1, 1024, 33)
    q, k, v = make_stripe_inputs(spec)
    say("[parity] causality")
    base = run_gpu(q, k, v, 256, 0.05)
    i = 600
    rng = np.random.default_rng(0)
    v2 = v.copy()
    v2[:, :, i + 1:] = rng.integers(0x3c00, 0x4000, size=v2[:, :, i + 1:].shape,
                                    dtype=np.uint16)
    pert = run_gpu(q, k, v2, 256, 0.05)
    assert np.array_equal(base["o"][:, :, :i + 1], pert["o"][:, :, :i + 1])
    assert not np.array_equal(base["o"][:, :, i + 1:], pert["o"][:, :, i + 1:])
    # keys of later segments change nothing in earlier segments
    k2 = k.copy()
    k2[:, :, 768:] = rng.integers(0x3c00, 0x4000, size=k2[:, :, 768:].shape,
                                  dtype=np.uint16)
    pert = run_gpu(q, k2, v, 256, 0.05)
    assert np.array_equal(base["o"][:, :, :768], pert["o"][:, :, :768])
    assert np.array_equal(base["n_I"][:, :, :12], pert["n_I"][:, :, :12])


def test_random_shapes():
    """Seeded random combinations of batch, heads per KV head (1-8, odd
    included), segment length (64-512, odd block counts included), segment
    count, tau and flags, each against the oracle as in test_parity_small."""
    rng = np.random.default_rng(2026)
    flagset = [0, 0, 0, O.SA_NO_QPERM, O.SA_NO_KVPERM, O.SA_SEGMENT_KV,
               O.SA_LOCAL_ONLY, O.SA_NO_EARLYSTOP,
               O.SA_SEGMENT_KV | O.SA_NO_QPERM]
    for c in range(24):
        B = int(rng.choice([1, 1, 2]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3, 4, 4, 8]))
        S = int(rng.choice([64, 128, 192, 256, 320, 512]))
        T = int(rng.integers(1, 7))
        while T > 1 and B * G * Hkv * S * T > 6 * 4096:
            T -= 1
        N = S * T
        tau = float(rng.choice([0.0, 0.005, 0.02, 0.1, 0.4]))
        flags = int(rng.choice(flagset))
        spec = StripeSpec(B, G * Hkv, Hkv, N, 128, n_vert=min(16, N // 16),
                          n_horiz=min(8, N // 32), window=min(64, N // 8),
                          seed=3000 + c)
        say(f"[random {c}] B={B} Hq={G * Hkv} Hkv={Hkv} N={N} S={S} "
            f"tau={tau} flags={flags}")
        q, k, v = make_stripe_inputs(spec)
        err, mse, nties, g, _, _ = _check_case(q, k, v, S, tau, flags)
        say(f"   max_abs={err:.3g} mse={mse:.3g} ties={nties}")


def test_parity_llama_layer_n32k_full_plan_sampled_outputs():
    """Llama-3.1-8B-shaped layer at N = 32768 (the 32K workload): every index
    array and every stop point against the oracle; outputs on 48 sampled
    query blocks (oracle row by row)."""
    cfg = get_config(2)
    q, k, v = make_stripe_inputs(cfg.spec)
    S, tau = cfg.segment, cfg.tau
    say("[parity] 32K workload: oracle plan")
    pl = O.plan(q, k, S)
    say("[parity] 32K workload: GPU")
    g = run_gpu(q, k, v, S, tau)
    assert_plan_equal(g, pl)
    say("[parity] 32K workload: oracle stop points (all blocks)")
    n_orc, traces = O.stop_points(q, k, pl, tau)
    ties = stop_mismatches(g["n_I"], n_orc, traces, tau)
    say(f"   ties={len(ties)} mean_n_I={g['n_I'].mean():.2f}")
    rng = np.random.default_rng(7)
    nb = q.shape[2] // 64
    blocks = [(0, int(h), int(I)) for h, I in zip(
        rng.integers(0, 32, 48), rng.integers(0, nb, 48))]
    blocks += [(0, 31, nb - 1), (0, 0, 0), (0, 5, nb // 2)]
    n_use = n_orc.copy()
    for b, h, I in ties:
        n_use[b, h, I] = g["n_I"][b, h, I]
    o_ref, lse_ref = O.attend(q, k, v, pl, n_use, blocks=blocks)
    err, mse = assert_outputs_close(g["o"], o_ref, g["lse"], lse_ref)
    say(f"   sampled blocks: max_abs={err:.3g} mse={mse:.3g}")


def _sampled_check(q, k, v, S, tau, flags, pl, label, n_blocks=24, seed=11,
                   all_stops=False):
    """One GPU run at full size against the oracle: every index array
    bit-exact, then stop points (of every block with all_stops, else of the
    sampled ones) and outputs of sampled query blocks (plus the first and
    last block of the last head)."""
    g = run_gpu(q, k, v, S, tau, flags)
    assert_plan_equal(g, pl)
    B, Hq, N = q.shape[:3]
    nb = N // 64
    rng = np.random.default_rng(seed)
    blocks = [(int(b), int(h), int(I)) for b, h, I in zip(
        rng.integers(0, B, n_blocks), rng.integers(0, Hq, n_blocks),
        rng.integers(0, nb, n_blocks))]
    blocks += [(B - 1, Hq - 1, nb - 1), (0, 0, 0)]
    if all_stops:
        say(f"   {label}: oracle stop points of all {B * Hq * nb} blocks")
        n_orc, traces = O.stop_points(q, k, pl, tau)
    else:
        n_orc, traces = O.stop_points(q, k, pl, tau, blocks=blocks)
    mask = n_orc >= 0
    gn = np.where(mask, g["n_I"], -1)
    ties = stop_mismatches(gn, n_orc, traces, tau)
    n_use = n_orc.copy()
    for b, h, I in ties:
        n_use[b, h, I] = g["n_I"][b, h, I]
    o_ref, lse_ref = O.attend(q, k, v, pl, n_use, blocks=blocks)
    err, mse = assert_outputs_close(g["o"], o_ref, g["lse"], lse_ref)
    say(f"   {label}: stop points compared {int(mask.sum())} ties={len(ties)}"
        f" mean_n_I={g['n_I'].mean():.2f} sampled max_abs={err:.3g} "
        f"mse={mse:.3g}")
    return g


_INPUTS = {}


def _inputs(cid):
    """The workload's inputs, generated once per workload for the tests of
    this module that use it (the previous workload's are dropped)."""
    if cid not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[cid] = make_stripe_inputs(get_config(cid).spec)
    return _INPUTS[cid]


def _full_runs():
    runs = []
    c3, c4, c5 = get_config(3), get_config(4), get_config(5)
    runs += [(3, c3.segment, t_, 0, t_ == c3.tau) for t_ in c3.taus]
    runs += [(4, S_, c4.tau, 0, S_ == 1024) for S_ in c4.segments]
    runs += [(5, c5.segment, c5.tau, 0, False),
             (5, c5.segment, c5.tau, O.SA_NO_QPERM, False)]
    return runs


@pytest.mark.parametrize("cid,S,tau,flags,all_stops", _full_runs(),
                         ids=[f"cfg{r[0]}-S{r[1]}-tau{r[2]}-flags{r[3]}"
                              for r in _full_runs()])
def test_parity_full_size(cid, S, tau, flags, all_stops):
    """The 128K Llama-shaped layer (every tau of its sweep; every stop point
    at tau = 0.005), the 128K Qwen-shaped layer (every segment length; every
    stop point at S = 1024) and the batch-4 64K layer (S2O and KV
    permutation only) at their full sizes in the launch configuration the
    benchmark times: index arrays bit-exact, stop points and outputs of
    sampled blocks."""
    cfg = get_config(cid)
    say(f"[full] workload {cfg.name}: inputs")
    q, k, v = _inputs(cid)
    say(f"[full] oracle plan S={S} flags={flags}")
    pl = O.plan(q, k, S, flags=flags)
    say(f"[full] GPU S={S} tau={tau} flags={flags}")
    _sampled_check(q, k, v, S, tau, flags, pl,
                   f"S={S} tau={tau} flags={flags}", all_stops=all_stops)


def test_parity_batch4_tau0_is_dense():
    """The batch-4 64K layer at tau = 0 against dense causal attention
    (float64 oracle) on sampled rows of three heads."""
    cfg = get_config(5)
    q, k, v = _inputs(5)
    say("[full] tau = 0 against dense attention on sampled rows")
    g = run_gpu(q, k, v, cfg.segment, 0.0)
    rng = np.random.default_rng(3)
    N = q.shape[2]
    rows = rng.integers(0, N, 12)
    for b, h in [(0, 0), (3, 31), (2, 17)]:
        od, ld = O.dense_causal(q, k, v, rows=rows, heads=[(b, h)])
        err = np.abs(g["o"][b, h, rows] - od[b, h, rows]).max()
        assert err <= 2e-2, err
        assert np.abs(g["lse"][b, h, rows] - ld[b, h, rows]).max() <= LSE_TOL


def _bits(x):
    return round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_local_heavy_outputs_in_4_8():
    """Values in [4, 8) (bf16 step 2^-5) and attention whose local window
    carries a large share of each row's mass (up to about a half): one
    rounding of the final value to bf16 costs up to 2^-6 here, which leaves
    little of the 2e-2 bound. The state the local pass hands to the sparse
    pass must not be rounded to bf16 on the way (rounding it there and
    again at the end reaches about 0.024), and the weights of the PV
    products must be finer than bf16 (2^-9 relative of values up to 8 is
    another 0.016 at worst; fp16 weights leave 0.002). Every row's query
    and key share a random direction (a strong diagonal), scaled by a."""
    rng = np.random.default_rng(44)
    N, d, S, tau = 2048, 128, 512, 0.01
    r = rng.standard_normal((N, d))
    r /= np.linalg.norm(r, axis=1, keepdims=True)
    worst = 0.0
    # the last case: values around 1, so that half-rows below and above the
    # magnitude from which the local pass hands over residuals meet in one
    # prefill
    for a, lo, hi in ((5.0, 4.0, 8.0), (7.0, 4.0, 8.0), (7.0, 0.5, 1.5)):
        q = _bits((a * r + 0.3 * rng.standard_normal((N, d)))[None, None])
        k = _bits((a * r + 0.3 * rng.standard_normal((N, d)))[None, None])
        v = _bits(np.minimum(lo + (hi - lo) * rng.random((1, 1, N, d)),
                             hi - 2.0 ** -5))
        say(f"[local heavy] a={a} values in [{lo}, {hi})")
        err, mse, nties, g, pl, n_orc = _check_case(q, k, v, S, tau, 0)
        # the share of the local window in each row's mass (oracle)
        pll = O.plan(q, k, S, flags=O.SA_LOCAL_ONLY)
        nl, _ = O.stop_points(q, k, pll, 0.0)
        _, l_loc = O.attend(q, k, v, pll, nl)
        _, l_all = O.attend(q, k, v, pl, n_orc)
        share = np.exp(l_loc - l_all)[0, 0, S:]
        say(f"   max_abs={err:.4g} mse={mse:.3g} local share mean "
            f"{share.mean():.3f} max {share.max():.3f}")
        assert share.mean() > 0.15 and share.max() > 0.4
        assert g["n_I"][0, 0, S // 64:].min() > 0
        worst = max(worst, err)
    say(f"   worst max_abs {worst:.4g} (one bf16 rounding in [4, 8): "
        f"{0.5 * 2.0 ** -5:.4g})")


def test_saturated_fixed_point_and_wide_pooled_query():
    """Inputs whose fixed-point images saturate (entries of magnitude >= 128
    map to -32768 / 32767) in queries and keys, with G N = 131072 query rows
    per KV head: the pooled query then has entries beyond +-2^32, so the key
    scores' int64 arithmetic on the GPU uses the high word of every factor.
    Logits stay moderate: the saturated query dimensions meet key entries
    of at most 8 / 256, the saturated key entries meet query entries of at
    most 4 / 256."""
    rng = np.random.default_rng(45)
    B, Hq, Hkv, N, d, S = 1, 8, 1, 16384, 128, 2048
    spec = _spec(B, Hq, Hkv, N, 46, n_vert=32, window=128)
    q, k, v = make_stripe_inputs(spec)
    qf = bf16_bits_to_float32(q).astype(np.float64)
    kf = bf16_bits_to_float32(k).astype(np.float64)
    qf[..., 0] = 200.0
    qf[..., 1] = -300.0
    qf[..., 2] = rng.integers(-4, 5, size=qf[..., 2].shape) / 256.0
    kf[..., 0] = rng.integers(-8, 9, size=kf[..., 0].shape) / 256.0
    kf[..., 1] = rng.integers(-8, 9, size=kf[..., 1].shape) / 256.0
    kf[..., 2] = 0.0
    hot = rng.choice(N, 64, replace=False)
    kf[0, 0, hot, 2] = rng.choice([-250.0, -130.0, 128.0, 255.0], size=64)
    q, k = _bits(qf), _bits(kf)
    fq = O.fixed_point(q)
    assert (fq[..., 0] == 32767).all() and (fq[..., 1] == -32768).all()
    assert (np.abs(O.fixed_point(k[0, 0, hot, 2])) >= 32767).all()
    pl = O.plan(q, k, S)
    assert np.abs(pl.pooled).max() >= 2 ** 32
    assert (pl.pooled[0, 0, :2] == [32767 * Hq * N, -32768 * Hq * N]).all()
    for tau in (0.005, 0.05):
        say(f"[saturated] tau={tau}")
        err, mse, nties, g, _, _ = _check_case(q, k, v, S, tau, 0)
        say(f"   max_abs={err:.3g} mse={mse:.3g} ties={nties} "
            f"mean_n_I={g['n_I'].mean():.2f}")


def test_stop_points_with_large_mean_logits():
    """Mean-pooled logits between about 75 and 180 (natural log units):
    exp of them overflows fp32 above about 88.7, but the running share of
    the stop rule does not depend on a common factor of the estimates, so
    the stop points must still match the oracle's (float64) ones. Queries
    and keys share one direction u, keys with one weight per 64 keys."""
    rng = np.random.default_rng(47)
    N, d, S = 4096, 128, 512
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    qf = 34.0 * u + rng.standard_normal((1, 2, N, d))
    w = np.repeat(rng.uniform(25.0, 60.0, size=N // 64), 64).reshape(
        1, 1, N, 1)
    kf = w * u + rng.standard_normal((1, 1, N, d))
    q, k = _bits(qf), _bits(kf)
    v = _bits(rng.standard_normal((1, 1, N, d)))
    qm = bf16_bits_to_float32(q).astype(np.float64).mean(axis=2)
    km = bf16_bits_to_float32(k).astype(np.float64)
    tm = km[0, 0].reshape(-1, 64, d).mean(axis=1)
    ml = (tm @ qm[0].T) / np.sqrt(d)
    say(f"[large logits] tile mean logits {ml.min():.1f} .. {ml.max():.1f}")
    assert ml.min() > 60.0 and ml.max() > 150.0
    for tau in (0.001, 0.01, 0.1):
        say(f"[large logits] tau={tau}")
        err, mse, nties, g, pl, n_orc = _check_case(q, k, v, S, tau, 0)
        full = np.repeat(np.arange(N // S) * (S // 64), S // 64)
        stopped = (g["n_I"][0] < full[None, :]).sum()
        say(f"   max_abs={err:.3g} mse={mse:.3g} ties={nties} "
            f"mean_n_I={g['n_I'].mean():.2f} blocks stopped early {stopped}")
        if tau >= 0.01:
            assert stopped > 0


def test_non_current_streams():
    """plan, prefill and forward on streams other than torch's current one
    (the binding records its workspace, inputs and outputs on the streams
    that use them) give the bits of the default path, also when the plan
    objects are dropped right after their last launch and new tensors are
    allocated on the current stream before anything has finished."""
    import torch
    import permuted_block_sparse_amd as pbs
    from tests.gpu_helpers import to_device
    spec = _spec(1, 4, 2, 4096, 48, n_vert=32, window=128)
    q, k, v = make_stripe_inputs(spec)
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    S, tau = 512, 0.05
    pl = pbs.plan(tq, tk, S, tau)
    o_ref, l_ref = pbs.prefill(pl, tq, tk, tv, return_lse=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    say("[streams] plan + prefill on a second stream")
    p1 = pbs.plan(tq, tk, S, tau, stream=s1)
    o1, l1 = pbs.prefill(p1, tq, tk, tv, return_lse=True, stream=s1)
    del p1
    junk = [torch.full((1 << 24,), 7, dtype=torch.int32, device="cuda:0")
            for _ in range(4)]
    say("[streams] forward on two other streams")
    pf, of, lf = pbs.forward(tq, tk, tv, S, tau, return_lse=True, stream=s1,
                             side_stream=s2)
    del pf
    junk += [torch.full((1 << 24,), 9, dtype=torch.int32, device="cuda:0")
             for _ in range(4)]
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l1, l_ref)
    assert torch.equal(of.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lf, l_ref)
    del junk


def _check_topk(q, k, v, S, K, flags=0):
    from tests.gpu_helpers import unpack_tile_mask
    pl = O.plan(q, k, S, flags=flags)
    n_ref, m_ref, _ = O.topk_selection(q, k, pl, K)
    g = run_gpu(q, k, v, S, 0.05, flags, topk=K)
    assert_plan_equal(g, pl)
    B, Hq, N = q.shape[:3]
    for b in range(B):
        for h in range(Hq):
            for I in range(N // 64):
                ntl = (I * 64 // S) * S // 64
                got = unpack_tile_mask(g["topk_masks"][b, h, I], ntl)
                assert np.array_equal(got, m_ref[(b, h, I)]), (K, b, h, I)
    assert np.array_equal(g["n_I"], n_ref), K
    o_ref, l_ref = O.attend(q, k, v, pl, n_ref, tile_mask=m_ref)
    err, mse = assert_outputs_close(g["o"], o_ref, g["lse"], l_ref)
    return err, mse, g, pl


TOPK_CASES = [
    # name, spec, S, Ks
    ("gqa_n1024_s256", _spec(1, 4, 2, 1024, 49), 256, (0, 1, 5, 12)),
    ("b2_n2048_s128", _spec(2, 2, 1, 2048, 51), 128, (3, 17)),
    # 9 tiles per segment: selections and tile chunks end mid-word
    ("ragged_s576_n2304", _spec(1, 4, 1, 2304, 52), 576, (2, 7, 30)),
    # 256 blocks per (KV head, segment): two scoring workgroups; up to 192
    # tiles per list: six tile chunks
    ("two_chunks_s4096_n16384", _spec(1, 4, 1, 16384, 53, n_vert=64,
                                      window=128), 4096, (40, 100)),
]


@pytest.mark.parametrize("name,spec,S,Ks", TOPK_CASES,
                         ids=[c[0] for c in TOPK_CASES])
def test_topk_parity(name, spec, S, Ks):
    """Per-block centroid Top-K: the GPU's selections (bitmasks over the
    positions of L_t) equal the oracle's bit for bit, n_I = min(K, t S /
    64), and outputs match the oracle on those selections."""
    q, k, v = make_stripe_inputs(spec)
    for K in Ks:
        say(f"[topk] {name} K={K}")
        err, mse, g, pl = _check_topk(q, k, v, S, K)
        say(f"   max_abs={err:.3g} mse={mse:.3g} mean_n_I="
            f"{g['n_I'].mean():.2f}")


def test_topk_worked_example_and_mode_changes():
    """The hand-derived selection on the GPU plan (head dimension padded to
    128): block 2 takes the e1 tile, block 3 the e2 tile, segment 2's
    zero-query blocks the first positions. K >= all gives dense attention;
    back to the tau stop with K < 0 the stop points are the oracle's again;
    injecting a KV order ends the mode."""
    import torch
    from tests.gpu_helpers import unpack_tile_mask, to_device
    import permuted_block_sparse_amd as pbs
    N, S = 384, 128
    qf = np.zeros((1, 1, N, 128), np.float32)
    qf[0, 0, :128, 0] = 1.0
    qf[0, 0, 128:192, 1] = 1.0
    qf[0, 0, 192:256, 0] = 1.0
    kf = np.zeros((1, 1, N, 128), np.float32)
    kf[0, 0, :64, 0] = 1.0
    kf[0, 0, 64:128, 1] = 1.0
    q, k = _bits(qf), _bits(kf)
    v = _bits(np.random.default_rng(54).standard_normal((1, 1, N, 128)))
    say("[topk] worked example")
    g = run_gpu(q, k, v, S, 0.05, topk=1)
    got = {I: unpack_tile_mask(g["topk_masks"][0, 0, I],
                               (I * 64 // S) * S // 64).astype(int).tolist()
           for I in range(2, 6)}
    assert got == {2: [1, 0], 3: [0, 1], 4: [1, 0, 0, 0], 5: [1, 0, 0, 0]}
    spec = _spec(1, 4, 2, 1024, 55)
    q, k, v = make_stripe_inputs(spec)
    say("[topk] K >= all is dense")
    od, ld = O.dense_causal(q, k, v)
    g = run_gpu(q, k, v, 256, 0.05, topk=1000)
    assert_outputs_close(g["o"], od, g["lse"], ld)
    say("[topk] back to the tau stop, then a KV order injection")
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    p = pbs.plan(tq, tk, 256, 0.05)
    p.set_topk(2)
    pbs.prefill(p, tq, tk, tv)
    assert (p.n_I()[:, :, 4:] == 2).all()
    p.set_topk(-1)
    o1 = pbs.prefill(p, tq, tk, tv)
    pl = O.plan(q, k, 256)
    n_tau, traces = O.stop_points(q, k, pl, 0.05)
    assert not stop_mismatches(p.n_I(), n_tau, traces, 0.05)
    p.set_topk(2)
    p.set_kv_order(torch.arange(1024, dtype=torch.int32,
                                device="cuda:0").repeat(1, 2, 1))
    pbs.prefill(p, tq, tk, tv)
    torch.cuda.synchronize()
    pli = O.plan(q, k, 256, kv_order=np.tile(np.arange(1024), (1, 2, 1)))
    n_i, tr_i = O.stop_points(q, k, pli, 0.05)
    assert not stop_mismatches(p.n_I(), n_i, tr_i, 0.05)


def test_random_shapes_selection_modes():
    """The fixed budget, the exact per-block maximum and the centroid Top-K
    on seeded random shapes (batch, heads per KV head 1-8, segments of
    64-512 with odd block counts), four of each, against the oracle."""
    rng = np.random.default_rng(2027)
    for c in range(12):
        B = int(rng.choice([1, 1, 2]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3, 4, 4, 8]))
        S = int(rng.choice([64, 128, 192, 256, 320, 512]))
        T = int(rng.integers(2, 7))
        while T > 2 and B * G * Hkv * S * T > 4 * 4096:
            T -= 1
        N = S * T
        spec = StripeSpec(B, G * Hkv, Hkv, N, 128, n_vert=min(16, N // 16),
                          n_horiz=min(8, N // 32), window=min(64, N // 8),
                          seed=4000 + c)
        q, k, v = make_stripe_inputs(spec)
        pl = O.plan(q, k, S)
        tag = f"B={B} Hq={G * Hkv} Hkv={Hkv} N={N} S={S}"
        mode = c % 3
        if mode == 0:
            K = int(rng.integers(0, 2 * N // 64))
            say(f"[random budget] K={K} {tag}")
            g = run_gpu(q, k, v, S, 0.05, budget=K)
            n_ref, _ = O.stop_points(q, k, pl, 0.05, budget=K)
            assert np.array_equal(g["n_I"], n_ref)
            o_ref, l_ref = O.attend(q, k, v, pl, n_ref)
            assert_outputs_close(g["o"], o_ref, g["lse"], l_ref)
        elif mode == 1:
            # a threshold in a gap of at least 2e-3 between the oracle's
            # tile maxima (fp32 and float64 maxima cannot disagree there)
            _, _, mx = O.exact_max_selection(q, k, pl, 0.0)
            vals = np.sort(np.concatenate([m for m in mx.values() if len(m)]))
            gaps = np.flatnonzero(np.diff(vals) >= 2e-3)
            if len(gaps):
                i = gaps[int(rng.integers(0, len(gaps)))]
                theta = float((vals[i] + vals[i + 1]) / 2)
            else:  # above every maximum: no sparse tile
                theta = float(vals[-1]) + 1.0
            say(f"[random exact] theta={theta:.4f} {tag}")
            g = run_gpu(q, k, v, S, 0.05, max_theta=theta)
            n_ref, masks, _ = O.exact_max_selection(q, k, pl, theta)
            assert np.array_equal(g["n_I"], n_ref)
            o_ref, l_ref = O.attend(q, k, v, pl, n_ref, tile_mask=masks)
            assert_outputs_close(g["o"], o_ref, g["lse"], l_ref)
        else:
            K = int(rng.integers(0, 2 * N // 64))
            say(f"[random topk] K={K} {tag}")
            _check_topk(q, k, v, S, K)
