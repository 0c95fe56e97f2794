"""Host logic of bench.py, no GPU: the one-GPU guard, the stop scan's tile
accounting and the planner's algorithmic byte model, each against a count
made another way (a simulation, the oracle's own lists, a direct count)."""
import math
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import s2o as O  # noqa: E402
from synthetic import StripeSpec, make_stripe_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _scan_simulated(n_I, B, Hq, Hkv, N, S, chunk=32):
    # one reader per (b, KV head, segment t >= 1) takes L_t chunk by chunk
    # and ends after the chunk in which the last of its blocks stops (a
    # block with n_I = n stops at tile n; n = t S / 64 never stops)
    T, bps, G = N // S, S // 64, Hq // Hkv
    total = 0
    for b in range(B):
        for g in range(Hkv):
            for t in range(1, T):
                ntl = t * bps
                ns = [int(n_I[b, h, t * bps + i])
                      for h in range(g * G, (g + 1) * G) for i in range(bps)]
                read = 0
                while read < ntl:
                    read = min(read + chunk, ntl)
                    if all(n < read for n in ns):
                        break
                total += read
    return total


def test_scan_tiles_read_matches_a_simulation():
    rng = np.random.default_rng(7)
    for B, Hq, Hkv, N, S in ((1, 2, 1, 4096, 512), (2, 4, 2, 8192, 1024),
                             (1, 8, 2, 16384, 2048)):
        T, bps = N // S, S // 64
        n_I = np.zeros((B, Hq, N // 64), dtype=np.int64)
        for t in range(1, T):
            ntl = t * bps
            # small stop points, a few that never stop, exact chunk edges
            v = rng.integers(0, ntl + 1, size=(B, Hq, bps))
            v[rng.random(v.shape) < 0.6] //= 7
            v[rng.random(v.shape) < 0.05] = ntl
            v[rng.random(v.shape) < 0.05] = min(31, ntl)
            n_I[..., t * bps:(t + 1) * bps] = v
        got = bench.scan_tiles_read(n_I, B, Hq, Hkv, N, S)
        assert got == _scan_simulated(n_I, B, Hq, Hkv, N, S)


def test_plan_bytes_restricted_lists_match_the_oracle():
    # the restriction's output is exactly the oracle's lists L_t (int32)
    spec = StripeSpec(1, 4, 2, 1024, 128, n_vert=4, n_horiz=2, window=32,
                      seed=3)
    q, k, _ = make_stripe_inputs(spec)
    S = 256
    pl = O.plan(q, k, S)
    B, Hq, Hkv, N, d = 1, 4, 2, 1024, 128
    res = bench.plan_kernel_bytes(B, Hq, Hkv, N, S, d, scan_tiles=0)
    nrc = -(-N // 4096)
    cnt = B * Hkv * nrc * (N // S) * 4
    written_lists = res["k_restrict_write"]["bytes"] - (B * Hkv * N * 4 + cnt)
    assert written_lists == pl.L.size * 4
    for t in range(1, N // S):
        assert len(O.restricted_list(pl, 0, 0, t)) == t * S


def test_plan_bytes_sort_dispatches():
    # merge passes double sorted runs of 4096 until one run holds the segment
    for N, S in ((131072, 2048), (12288, 6144), (8192, 4096), (2048, 512)):
        res = bench.plan_kernel_bytes(1, 32, 8, N, S, 128, scan_tiles=0)
        want = sum(math.ceil(math.log2(-(-L // 4096))) if L > 4096 else 0
                   for L in (N, S))
        got = res.get("k_merge_pass", {"dispatches": 0})["dispatches"]
        assert got == want, (N, S, got, want)
        # one chunk-sort workgroup per 4096 keys (or per shorter segment)
        assert res["k_chunk_sort[pi_K]"]["workgroups"] == 8 * -(-N // 4096)
        assert (res["k_chunk_sort[pi_Q]"]["workgroups"]
                == 32 * (N // S) * -(-S // 4096))


def test_plan_bytes_streaming_passes_read_each_operand_once():
    B, Hq, Hkv, N, S, d = 1, 32, 8, 131072, 2048, 128
    res = bench.plan_kernel_bytes(B, Hq, Hkv, N, S, d, scan_tiles=0)
    q_bytes = B * Hq * N * d * 2
    k_bytes = B * Hkv * N * d * 2
    # pooling, query score and block sums each read all of Q once; the key
    # score reads all of K once; the rest of each figure is small outputs
    for name in ("k_pool_q", "k_query_score", "k_block_qsum"):
        assert q_bytes <= res[name]["bytes"] < 1.1 * q_bytes, name
    assert k_bytes <= res["k_key_score"]["bytes"] < 1.2 * k_bytes


def test_selection_stats_match_the_oracle_metrics():
    # the bench's pair sparsity and tile density (from n_I and pi_Q alone)
    # against the oracle's definitions (explicit per-row selected sets and
    # per-block local tiles), on plans with a permuted and an identity
    # query order, stop points that differ per block, and two batches
    spec = StripeSpec(2, 4, 2, 1024, 128, n_vert=4, n_horiz=2, window=32,
                      seed=5)
    q, k, _ = make_stripe_inputs(spec)
    S = 256
    for flags, tau in ((0, 0.05), (0, 0.0), (O.SA_NO_QPERM, 0.2),
                       (O.SA_LOCAL_ONLY, 0.0)):
        pl = O.plan(q, k, S, flags=flags)
        n_I, _ = O.stop_points(q, k, pl, tau)
        want = O.metrics(pl, n_I)
        got = bench.selection_stats(n_I, 1024, S, pl.pi_q)
        assert abs(got["pair_sparsity"] - want["pair_sparsity"]) < 1e-12
        assert abs(got["tile_density"] - want["tile_density"]) < 1e-12
        assert got["visited_sparse_tiles"] == want["visited_sparse_tiles"]
        assert got["local_tiles_touched"] == want["visited_diag_tiles"]
        if tau == 0.05:
            assert 0.0 < got["pair_sparsity"] < 1.0
