#!/usr/bin/env python3
"""Benchmark: permuted early-stopping block-sparse prefill attention, 128K.

One step = the whole hot path on one attention layer of the Llama-3.1-8B
shape at N = 131072 (32 query heads, 8 KV heads, d = 128, bf16, causal), in
one sparse_attn_forward call: the plan (pooling, scores, both orders,
restricted lists, stop points) on the launch stream while the dense local
windows run on a second stream, then the sparse tiles with the tau stop and
the scatter; inputs resident in HBM. Prints ONE JSON line (rank 0, one
GPU). The plan alone, the prefill alone and the two calls in order on one
stream are timed as well.

Besides the timed steps the run reports: the stop statistics (pair sparsity,
tile density, visited tiles), MSE and attention recall against dense
attention (the same kernel at tau = 0, itself checked against the float64
oracle), the tau sweep of the workload, the variants at matched sparsity
(uniform tile budget, per-block centroid Top-K, exact per-block maximum
test), the segment-local KV order, planner overhead, the attention kernel's
MFMA roofline, the other workloads (the tiny case, the 32K layer, the 128K
Qwen-shaped layer over its segment lengths, the batch-4 64K ablation), and
the CPU oracle timed on the host's cores on a bounded sample, which also
checks the GPU run on that sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0
TILE_FLOP = 4 * 64 * 64 * 128  # QK^T + PV of one 64 x 64 tile, d = 128
METRIC = "ms/layer sparse prefill attn @128K; sparsity & MSE; MFMA util vs bf16 peak"
# query blocks and dense rows in the CPU oracle's timed sample
CPU_SAMPLE_BLOCKS = 240
CPU_SAMPLE_ROWS = 512
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_fwd_traffic_n128k.json")
ATTN_SOURCE = os.path.join(ROOT, "permuted_block_sparse_amd", "csrc",
                           "attn_kernel.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3,
                    help="workload id (3 = Llama-3.1-8B layer at 128K)")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--segment", type=int, default=None)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the reports of the other workloads")
    ap.add_argument("--profile-once", action="store_true",
                    help="one plan + one prefill, no timing (counter runs)")
    ap.add_argument("--plan-only", type=int, default=0, metavar="K",
                    help="only K plans after one warm-up plan (planner "
                         "kernel traces; no attention)")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="K",
                    help="one plan, then K prefills of it after one warm-up "
                         "prefill (attention kernel traces; no planner "
                         "kernel runs beside them)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    metavar="MIB",
                    help="only copy MIB MiB device->device (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    return ap.parse_args()


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path "
              "(the method would shard over independent KV heads with no "
              "communication between GPUs). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import permuted_block_sparse_amd as pbs
    from synthetic import get_config, make_stripe_inputs

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes device to device")
        return

    cfg = get_config(args.config)
    spec = cfg.spec
    S = args.segment or cfg.segment
    tau = cfg.tau if args.tau is None else args.tau
    B, Hq, Hkv, N, d = (spec.batch, spec.heads_q, spec.heads_kv,
                        spec.seq_len, spec.head_dim)
    dev = torch.device("cuda:0")
    log(f"[bench] workload {cfg.name}: generating inputs")
    t0 = time.time()
    q, k, v = make_stripe_inputs(spec)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; uploading")

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    tq, tk, tv = up(q), up(k), up(v)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority, like every stream here
    out = torch.empty_like(tq)

    def step(t_=tau):
        # the whole path in one call: the planner on `stream`, the dense
        # local windows on `side` meanwhile, then the sparse tiles
        return pbs.forward(tq, tk, tv, S, t_, out=out, side_stream=side)[0]

    if args.profile_once:
        step()
        torch.cuda.synchronize()
        log("[bench] one plan + prefill done")
        return
    if args.plan_only:
        for i in range(args.plan_only + 1):
            pbs.plan(tq, tk, S, tau)
            torch.cuda.synchronize()
        log(f"[bench] {args.plan_only} plans done")
        return
    if args.prefill_only:
        pl = pbs.plan(tq, tk, S, tau)
        pbs.prefill(pl, tq, tk, tv, out=out)
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.prefill_only):
            a_ = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            pbs.prefill(pl, tq, tk, tv, out=out)
            b_.record(stream)
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_))
        log(f"[bench] {args.prefill_only} prefills alone: mean "
            f"{float(np.mean(ts)):.3f} ms (HIP events)")
        return

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        pl = step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step")

    # The attention launches' duration (the roofline's kernel): HIP events
    # around each prefill of the last step's plan, on the launch stream,
    # right after the timed steps (inside a fused step the attention
    # launches interleave with the planner's).
    pre_ev = [(torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for a_, b_ in pre_ev:
        a_.record(stream)
        pbs.prefill(pl, tq, tk, tv, out=out)
        b_.record(stream)
    torch.cuda.synchronize()
    attn_launch_ms = [a_.elapsed_time(b_) for a_, b_ in pre_ev]
    attn_mean = float(np.mean(attn_launch_ms))
    log(f"[bench] prefill launch {attn_mean:.3f} ms")

    # ---- stage split with HIP events on the launch stream
    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)), float(np.mean(ts))

    plan_ms, _ = timed(lambda: pbs.plan(tq, tk, S, tau), max(3, args.steps))

    def plan_then_prefill():
        pbs.prefill(pbs.plan(tq, tk, S, tau), tq, tk, tv, out=out)
    seq_ms, _ = timed(plan_then_prefill, max(3, args.steps))
    pl = pbs.plan(tq, tk, S, tau)
    attn_med = float(np.median(attn_launch_ms))
    n_I = pl.n_I()
    log(f"[bench] plan {plan_ms:.3f} ms, prefill {attn_med:.3f} ms, "
        f"plan then prefill {seq_ms:.3f} ms")

    T = N // S
    nb = N // 64
    # visited local tiles: the local pass takes every segment's rows in
    # their own order, block i of a segment against its key blocks 0 .. i
    # (the last one masked), so bps (bps + 1) / 2 tiles per segment and head
    bps = S // 64
    diag_tiles = B * Hq * T * bps * (bps + 1) // 2
    sparse_tiles = int(n_I.sum())
    visited = diag_tiles + sparse_tiles
    flop_launch = visited * TILE_FLOP
    achieved = flop_launch / (attn_mean * 1e-3) / 1e12
    sel_stats = selection_stats(n_I, N, S, pl.pi_q())
    dense_flop = 4.0 * d * N * (N + 1) / 2 * B * Hq

    result = {
        "metric": METRIC,
        "value": round(ms_step, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic stripe-structured Q/K/V (seeded), random-init "
                "stand-in for a Llama-3.1-8B attention layer",
        "config": {"workload": cfg.name, "batch": B, "heads_q": Hq,
                   "heads_kv": Hkv, "seq_len": N, "head_dim": d,
                   "segment": S, "block": 64, "tau": tau,
                   "parallelism": "single GPU"},
        "stages_ms": {"plan": round(plan_ms, 4),
                      "prefill": round(attn_med, 4),
                      "overhead_frac": round(plan_ms / attn_med, 4),
                      "plan_then_prefill_one_stream": round(seq_ms, 4),
                      "step_fused": round(ms_step, 4)},
        "stop": {"pair_sparsity": round(sel_stats["pair_sparsity"], 5),
                 "tile_density": round(sel_stats["tile_density"], 5),
                 "mean_n_I": round(float(n_I.mean()), 2),
                 "visited_sparse_tiles": sparse_tiles,
                 "visited_local_tiles": diag_tiles,
                 "dense_equiv_tflops": round(dense_flop / attn_med / 1e9, 1),
                 "visited_tile_tflops": round(achieved, 1)},
        "plan_bytes": plan_kernel_bytes(
            B, Hq, Hkv, N, S, d,
            scan_tiles_read(n_I, B, Hq, Hkv, N, S) if tau > 0 else 0,
            scanning=tau > 0),
    }
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("source_sha256_16") == source_hash(ATTN_SOURCE)
                and tr.get("workload") == cfg.name and tr.get("tau") == tau):
            traffic = tr.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    result["roofline"] = {
        "bound": "mfma", "achieved": round(achieved, 2),
        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": traffic,
        "kernel": "k_attn_fwd (kLocal + kFastRef + kMaxRef launches of a prefill)",
        "flop_per_launch": flop_launch,
        "avg_launch_ms": round(attn_mean, 4)}

    gpu = None
    if not args.no_cpu_baseline:
        # the GPU results the oracle's sample is checked against (the step's
        # plan and output at the workload's tau; the dense run at tau = 0)
        G = Hq // Hkv
        import torch
        o_dense = torch.empty_like(tq)
        pl0 = pbs.plan(tq, tk, S, 0.0)
        pbs.prefill(pl0, tq, tk, tv, out=o_dense)
        pbs.prefill(pl, tq, tk, tv, out=out)
        gpu = {"n_I": n_I, "pi_k": pl.pi_k()[:1, :1],
               "pi_q": pl.pi_q()[:1, :G],
               "L": pl.restricted_lists()[:1, :1],
               "o": bf16_to_f64(out[:1, :G]),
               "o_dense": bf16_to_f64(o_dense[:1, :1])}
        del o_dense, pl0
    if not args.no_extras:
        result.update(extras(args, cfg, tq, tk, tv, S, tau))
        if not args.no_other_workloads:
            del out
            result["workloads"] = workload_reports()
    if gpu is not None:
        result["cpu_baseline"] = cpu_baseline(cfg, q, k, v, S, tau, gpu)
    print(json.dumps(result), flush=True)


def bf16_to_f64(t):
    import torch
    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def selection_stats(n_I, N, S, pi_q=None):
    """Pair sparsity and tile density of a selection (S2O page, Key points:
    sparsity is the share of causal query-key pairs skipped, density its
    complement; the tile density counts the 64 x 64 tiles a selection
    touches, for performance accounting).

    n_I: [B, Hq, N / 64], the tiles of L_t each query block attends;
    pi_q: [B, Hq, N], the query order (needed for the tile density's local
    tiles; None: no tile density). A row of segment t sees the keys of its
    own segment up to itself (S (S + 1) / 2 pairs per segment and head) and
    the 64 keys of each of its block's tiles (64 rows: 4096 pairs a tile).
    A block touches local block c of its segment when its largest row
    reaches the block's first key, i.e. blocks 0 .. (max row - t S) // 64.
    """
    n_I = np.asarray(n_I)
    B, Hq, nb = n_I.shape
    T = N // S
    far = float(n_I.sum())
    sel = B * Hq * T * S * (S + 1) / 2 + 4096.0 * far
    out = {"pair_sparsity": 1.0 - sel / (B * Hq * N * (N + 1) / 2),
           "visited_sparse_tiles": int(far)}
    if pi_q is not None:
        top = np.asarray(pi_q).reshape(B, Hq, nb, 64).max(axis=-1)
        seg0 = (np.arange(nb) * 64) // S * S
        local = int(((top - seg0) // 64 + 1).sum())
        out["tile_density"] = (local + far) / (B * Hq * nb * (nb + 1) / 2)
        out["local_tiles_touched"] = local
    return out


def scan_tiles_read(n_I, B, Hq, Hkv, N, S, chunk=32):
    """Key tiles of L_t whose sums the stop scan gathers: one workgroup per
    (b, KV head, segment t >= 1) reads L_t in chunks of 32 tiles until every
    block of its G heads has stopped (a block that never stops reads all
    t S / 64 tiles)."""
    T, bps, G = N // S, S // 64, Hq // Hkv
    mx = n_I.reshape(B, Hkv, G, T, bps).max(axis=(2, 4))  # (B, Hkv, T)
    total = 0
    for t in range(1, T):
        ntl = t * bps
        m = mx[:, :, t]
        total += int(np.minimum((m // chunk + 1) * chunk, ntl).sum())
    return total


def plan_kernel_bytes(B, Hq, Hkv, N, S, d, scan_tiles, scanning=True):
    """Algorithmic HBM bytes of each planner kernel in one plan: every
    operand read once, every result written once; gathers count the rows
    and index entries they fetch. Returns {kernel: {"bytes": per plan,
    "dispatches": per plan}}; the two chunk-sort dispatches are told apart
    by their workgroup count."""
    T, nb, bps = N // S, N // 64, S // 64
    row = 2 * d
    qb, kb = B * Hq * N * row, B * Hkv * N * row
    npc = -(-N // 1024)
    nrc = -(-N // 4096)
    part = B * Hq * npc * d * 8
    out = {}
    out["k_pool_q"] = qb + part
    out["k_pool_reduce"] = part + B * Hkv * d * 8
    out["k_key_score"] = (kb + B * Hkv * d * 8 + B * Hkv * N * 8
                          + B * Hkv * nb * d * 4)
    out["k_segment_sum"] = B * Hkv * nb * d * 4 + B * Hkv * T * d * 8
    out["k_contrast"] = (B * Hkv * (T - 1) * 64 * (row + 4)
                         + 2 * B * Hkv * T * d * 8)
    out["k_query_score"] = qb + B * Hkv * T * d * 8 + B * Hq * N * 8
    res = {k_: {"bytes": v_, "dispatches": 1} for k_, v_ in out.items()}

    def sort(name, n_seg, seglen, score_b):
        chunk = min(seglen, 4096)
        nch = -(-seglen // chunk)
        n = n_seg * seglen
        passes = 0
        w = chunk
        while w < seglen:
            passes += 1
            w *= 2
        # chunk sort: scores in; keys + indices out (indices only when one
        # chunk holds the segment); each merge pass: keys + indices in and
        # out (indices only from the last pass)
        res[f"k_chunk_sort[{name}]"] = {
            "bytes": n * (score_b + (4 if passes == 0 else 12)),
            "dispatches": 1, "workgroups": n_seg * nch}
        return passes, n

    pk, nk = sort("pi_K", B * Hkv, N, 8)
    pq, nq = sort("pi_Q", B * Hq * T, S, 8)
    mb = sum(n * (24 * (p - 1) + 16) for p, n in ((pk, nk), (pq, nq)) if p)
    if pk + pq:
        res["k_merge_pass"] = {"bytes": mb, "dispatches": pk + pq}
    cnt = B * Hkv * nrc * T * 4
    L_bytes = B * Hkv * S * T * (T - 1) // 2 * 4
    res["k_restrict_count"] = {"bytes": B * Hkv * N * 4 + cnt, "dispatches": 1}
    res["k_restrict_scan"] = {"bytes": 2 * cnt, "dispatches": 1}
    res["k_restrict_write"] = {"bytes": B * Hkv * N * 4 + cnt + L_bytes,
                               "dispatches": 1}
    res["k_block_qsum"] = {"bytes": B * Hq * N * 4 + qb + B * Hq * nb * d * 4,
                           "dispatches": 1}
    # blocks that scan (t >= 1; none when a fixed count decides): their
    # query sums and pi_Q rows, the local segment's keys once per (b, KV
    # head, t), the gathered tiles' keys and L entries; n_I written
    sb = B * Hq * (T - 1) * bps if scanning else 0
    local = B * Hkv * (T - 1) * S * row if scanning else 0
    res["k_stop_scan"] = {
        "bytes": (sb * (d * 4 + 64 * 4) + local
                  + scan_tiles * 64 * (row + 4) + B * Hq * nb * 4),
        "dispatches": 1, "scan_tiles": scan_tiles}
    return res


def kernel_tiles(n_I, B, Hq, N, S):
    """64 x 64 tiles the attention kernel computes in one prefill: the local
    pass takes every segment's rows in their own order, block i of a
    segment against its key blocks 0 .. i (bps (bps + 1) / 2 tiles per
    segment and head), and the sparse pass n_I tiles per block."""
    bps, T = S // 64, N // S
    return B * Hq * T * bps * (bps + 1) // 2 + int(np.asarray(n_I).sum())


def hip_ms(fn, reps):
    """Median of `reps` calls of fn, timed by HIP events on torch's current
    stream (the stream every launch of fn goes to)."""
    import torch
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def recall_stats(lse_sel, lse_dense):
    """Share of each row's dense causal attention mass on its selected set:
    exp(lse over Sel(i) - lse over every causal key)."""
    import torch
    r = torch.exp(lse_sel - lse_dense)
    per_head = r.mean(dim=(0, 2))
    return {"recall_mean": float("%.4g" % r.mean().item()),
            "recall_min": float("%.4g" % r.min().item()),
            "recall_head_mean_min": float("%.4g" % per_head.min().item())}


def error_stats(o, ref, per_head=False):
    """MSE (and max-abs) of o against ref over every element; per query head
    when asked."""
    diff = o.float() - ref.float()
    sq = diff * diff
    out = {"mse_vs_dense": float(sq.mean().item()),
           "max_abs_vs_dense": float(diff.abs().max().item())}
    ph = sq.mean(dim=(0, 2, 3)).cpu().numpy()
    out["mse_per_head_max"] = float(ph.max())
    if per_head:
        out["mse_per_head"] = [float("%.3g" % x) for x in ph]
    return out


def measure(tq, tk, tv, S, tau, flags=0, setup=None, dense=None,
            reps=3, fused=False, per_head=False):
    """One selection on resident inputs: prefill time (HIP events, median of
    `reps`), selection statistics, the attention kernel's visited-tile rate
    and roofline fraction, and against `dense` ((o, lse) of the tau = 0 run)
    the MSE and the attention recall. setup(plan) applies a setter (budget,
    Top-K, threshold) before the prefills; fused also times the plan alone
    and the whole step (sparse_attn_forward, local windows on a second
    stream)."""
    import torch
    import permuted_block_sparse_amd as pbs
    B, Hq, N, d = tq.shape
    res = {"segment": S, "tau": tau, "flags": flags}
    if fused:
        side = torch.cuda.Stream()
        res["plan_ms"] = round(hip_ms(
            lambda: pbs.plan(tq, tk, S, tau, flags=flags), reps), 4)
        o_f = torch.empty_like(tq)
        pbs.forward(tq, tk, tv, S, tau, flags=flags, out=o_f,
                    side_stream=side)
        res["step_ms"] = round(hip_ms(
            lambda: pbs.forward(tq, tk, tv, S, tau, flags=flags, out=o_f,
                                side_stream=side), reps), 4)
        del o_f
    pl = pbs.plan(tq, tk, S, tau, flags=flags)
    if setup is not None:
        res["setup_ms"] = round(hip_ms(lambda: setup(pl), 1), 4)
    o = torch.empty_like(tq)
    pbs.prefill(pl, tq, tk, tv, out=o)   # rescans after a setter
    ms = hip_ms(lambda: pbs.prefill(pl, tq, tk, tv, out=o), reps)
    _, lse = pbs.prefill(pl, tq, tk, tv, out=o, return_lse=True)
    n_I = pl.n_I()
    st = selection_stats(n_I, N, S, pl.pi_q())
    tiles = kernel_tiles(n_I, B, Hq, N, S)
    tflops = tiles * TILE_FLOP / (ms * 1e-3) / 1e12
    res.update({"prefill_ms": round(ms, 4),
                "pair_sparsity": round(st["pair_sparsity"], 5),
                "tile_density": round(st["tile_density"], 5),
                "mean_n_I": round(float(n_I.mean()), 2),
                "visited_sparse_tiles": st["visited_sparse_tiles"],
                "kernel_tiles": tiles,
                "visited_tile_tflops": round(tflops, 1),
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4)})
    if dense is not None:
        res.update(error_stats(o, dense[0], per_head))
        res.update(recall_stats(lse, dense[1]))
    return res, pl, o, lse


def dense_reference(tq, tk, tv, S, flags=0):
    """The same kernel at tau = 0 visits every tile: dense causal attention
    (checked against the float64 oracle by the GPU tests). Returns
    (o, lse, prefill ms)."""
    import torch
    import permuted_block_sparse_amd as pbs
    pl = pbs.plan(tq, tk, S, 0.0, flags=flags)
    o = torch.empty_like(tq)
    pbs.prefill(pl, tq, tk, tv, out=o)
    ms = hip_ms(lambda: pbs.prefill(pl, tq, tk, tv, out=o), 2)
    _, lse = pbs.prefill(pl, tq, tk, tv, out=o, return_lse=True)
    return o, lse, ms


def matched_budget(n_tau_total, B, Hq, N, S):
    """Smallest uniform tile count K whose visited tiles (min(K, t S / 64)
    per block of segment t) reach n_tau_total."""
    T, bps = N // S, S // 64
    caps = np.repeat(np.arange(T) * bps, B * Hq * bps)
    lo, hi = 0, int(caps.max())
    while lo < hi:
        mid = (lo + hi) // 2
        if int(np.minimum(caps, mid).sum()) >= n_tau_total:
            hi = mid
        else:
            lo = mid + 1
    return lo


def extras(args, cfg, tq, tk, tv, S, tau):
    """The headline workload's sweeps and variants: tau sweep against dense
    attention, dense local window only, and at matched sparsity the fixed
    budget, the per-block centroid Top-K and the exact per-block maximum
    test; the segment-local KV order."""
    import permuted_block_sparse_amd as pbs
    B, Hq, N, d = tq.shape
    res = {}
    o_d, l_d, dense_ms = dense_reference(tq, tk, tv, S)
    dense = (o_d, l_d)
    log(f"[bench] tau=0 (dense) prefill {dense_ms:.3f} ms")
    sweep = []
    for t_ in sorted(set(cfg.taus) | {tau}):
        r, *_ = measure(tq, tk, tv, S, t_, dense=dense)
        r["speedup_vs_dense"] = round(dense_ms / r["prefill_ms"], 3)
        sweep.append(r)
        log(f"[bench] tau={t_}: {r['prefill_ms']:.3f} ms sparsity="
            f"{r['pair_sparsity']:.4f} mse={r['mse_vs_dense']:.3g}")
    res["tau_sweep"] = sweep
    res["dense_prefill_ms"] = round(dense_ms, 4)
    res["no_early_stop"] = {"note": "SA_NO_EARLYSTOP visits every tile: "
                                    "the tau = 0 run",
                            "prefill_ms": round(dense_ms, 4)}
    r, *_ = measure(tq, tk, tv, S, tau, flags=pbs.SA_LOCAL_ONLY, dense=dense)
    res["local_window_only"] = r
    log(f"[bench] local window only: {r}")

    # matched sparsity: the uniform budget and the per-block Top-K get the
    # smallest K whose visited tiles reach the tau stop's
    base = [x for x in sweep if x["tau"] == tau][0]
    n_tau = base["visited_sparse_tiles"]
    K = matched_budget(n_tau, B, Hq, N, S)
    r, *_ = measure(tq, tk, tv, S, tau, setup=lambda p: p.set_budget(K),
                    dense=dense)
    r.update({"budget_tiles": K, "tau_visited_tiles": n_tau})
    res["fixed_budget_matched"] = r
    log(f"[bench] fixed budget (matched): {r}")
    r, *_ = measure(tq, tk, tv, S, tau, setup=lambda p: p.set_topk(K),
                    dense=dense)
    r.update({"topk_tiles": K, "tau_visited_tiles": n_tau,
              "note": "setup_ms: exact scoring of every tile of every L_t "
                      "(fp64 MFMA) and the per-block selection"})
    res["topk_centroid_matched"] = r
    log(f"[bench] per-block centroid Top-K (matched): {r}")

    # exact per-block max test: theta bisected until the attended tiles
    # match the tau stop's
    pl = pbs.plan(tq, tk, S, tau)
    o = torch_empty_like(tq)

    def exact_count(theta):
        pl.set_max_threshold(theta)
        pbs.prefill(pl, tq, tk, tv, out=o)
        return int(pl.n_I().sum())
    lo_t, hi_t = 0.0, 4.0
    while exact_count(hi_t) > n_tau:
        hi_t *= 2.0
    while exact_count(lo_t) < n_tau:
        lo_t -= 4.0
    for _ in range(16):
        mid = 0.5 * (lo_t + hi_t)
        if exact_count(mid) >= n_tau:
            lo_t = mid
        else:
            hi_t = mid
    del pl, o
    r, *_ = measure(tq, tk, tv, S, tau,
                    setup=lambda p: p.set_max_threshold(lo_t), dense=dense)
    T, bps = N // S, S // 64
    r.update({"theta": round(lo_t, 5), "tau_visited_tiles": n_tau,
              "scored_tiles": int(sum(B * Hq * bps * t * bps
                                      for t in range(T)))})
    res["exact_max_matched"] = r
    log(f"[bench] exact max test (matched): {r}")

    r, *_ = measure(tq, tk, tv, S, tau, flags=pbs.SA_SEGMENT_KV, dense=dense,
                    fused=True)
    res["segment_kv_order"] = r
    log(f"[bench] segment-local KV order: {r}")
    return res


def torch_empty_like(x):
    import torch
    return torch.empty_like(x)


def upload(x):
    import torch
    return torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def workload_reports():
    """The other workloads at their full sizes, each on its own inputs: the
    tiny causal case, the 32K Llama-shaped layer, the 128K Qwen-shaped layer
    over its segment lengths (per-head MSE), and the batch-4 64K ablation
    (full S2O, KV permutation only, tau = 0 against plain dense attention
    with the identity orders)."""
    import torch
    import permuted_block_sparse_amd as pbs
    from synthetic import get_config, make_stripe_inputs
    out = {}
    for cid in (1, 2, 4, 5):
        cfg = get_config(cid)
        t0 = time.time()
        q, k, v = make_stripe_inputs(cfg.spec)
        log(f"[bench] workload {cfg.name}: inputs in {time.time() - t0:.1f}s")
        tq, tk, tv = upload(q), upload(k), upload(v)
        del q, k, v
        o_d, l_d, dense_ms = dense_reference(tq, tk, tv, cfg.segment)
        rep = {"workload": cfg.name, "shape": list(tq.shape),
               "dense_prefill_ms": round(dense_ms, 4), "runs": []}
        if cid == 4:
            runs = [(S_, cfg.tau, 0) for S_ in cfg.segments]
        elif cid == 5:
            runs = [(cfg.segment, cfg.tau, 0),
                    (cfg.segment, cfg.tau, pbs.SA_NO_QPERM)]
        else:
            runs = [(cfg.segment, cfg.tau, 0)]
        for S_, t_, fl in runs:
            r, *_ = measure(tq, tk, tv, S_, t_, flags=fl, dense=(o_d, l_d),
                            fused=True, per_head=(cid == 4))
            r["speedup_vs_dense"] = round(dense_ms / r["prefill_ms"], 3)
            if cid == 5:
                r["variant"] = "kv_perm_only" if fl else "s2o"
            rep["runs"].append(r)
            log(f"[bench] {cfg.name} S={S_} tau={t_} flags={fl}: "
                f"{r['prefill_ms']:.3f} ms sparsity {r['pair_sparsity']:.4f}"
                f" mse {r['mse_vs_dense']:.3g}")
        if cid == 5:
            # tau = 0 with the method's orders against plain dense causal
            # flash attention (identity orders): the same attention up to
            # the order in which each row's keys are added
            o_i, l_i, ms_i = dense_reference(
                tq, tk, tv, cfg.segment,
                flags=pbs.SA_NO_QPERM | pbs.SA_NO_KVPERM)
            diff = (o_d.float() - o_i.float())
            rep["tau0_vs_identity_order_dense"] = {
                "variant": "tau0", "prefill_ms": round(dense_ms, 4),
                "identity_order_prefill_ms": round(ms_i, 4),
                "max_abs": float(diff.abs().max().item()),
                "mse": float((diff * diff).mean().item()),
                "lse_max_abs": float((l_d - l_i).abs().max().item())}
            log(f"[bench] tau=0 vs identity-order dense: "
                f"{rep['tau0_vs_identity_order_dense']}")
            del o_i, l_i
        out[cfg.name] = rep
        del tq, tk, tv, o_d, l_d
        torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, q, k, v, S, tau, gpu):
    """The oracle, as it stands, on a bounded sample of the workload, timed
    in three parts on the host's cores (BLAS threads pinned to the cores the
    process may use): the plan of one KV group (integer ranking), the stop
    points and attention of CPU_SAMPLE_BLOCKS seeded random query blocks of
    that group, and dense causal attention of CPU_SAMPLE_ROWS seeded rows of
    one head; each extrapolated linearly to the layer (plan x KV groups,
    attention x query blocks, dense x rows). The same sample checks the GPU
    run (`gpu`: plan exports, stop points, outputs and the tau = 0 output):
    plan bit-exact, stop points equal up to near-tau ties, outputs within
    2e-2 max-abs and 1e-4 MSE."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
        blas = max([i.get("num_threads", 1) for i in threadpool_info()]
                   or [1])
    except Exception:
        limiter, blas = None, None
    spec = cfg.spec
    G = spec.heads_q // spec.heads_kv
    qs = np.ascontiguousarray(q[:1, :G])
    ks = np.ascontiguousarray(k[:1, :1])
    vs = np.ascontiguousarray(v[:1, :1])
    N = spec.seq_len
    nb = N // 64
    log("[bench] cpu baseline: oracle plan of one KV group")
    t0 = time.perf_counter()
    ref = O.plan(qs, ks, S)
    t_plan = time.perf_counter() - t0
    rng = np.random.default_rng(1)
    blocks = [(0, int(h), int(I)) for h, I in
              zip(rng.integers(0, G, CPU_SAMPLE_BLOCKS),
                  rng.integers(0, nb, CPU_SAMPLE_BLOCKS))]
    blocks.append((0, 0, nb - 1))
    log(f"[bench] cpu baseline: oracle stop points + attention of "
        f"{len(blocks)} blocks")
    t0 = time.perf_counter()
    n_ref, traces = O.stop_points(qs, ks, ref, tau, blocks=blocks)
    t_stop = time.perf_counter() - t0
    n_use = n_ref.copy()
    ties = 0
    n_gpu = gpu["n_I"][:1, :G]
    for b, h, I in blocks:
        if n_gpu[b, h, I] != n_ref[b, h, I]:
            m = int(min(n_gpu[b, h, I], n_ref[b, h, I]))
            if abs(traces[(b, h, I)][m] - tau) <= 1e-4 * tau:
                ties += 1
                n_use[b, h, I] = n_gpu[b, h, I]
    t0 = time.perf_counter()
    o_ref, _ = O.attend(qs, ks, vs, ref, n_use, blocks=blocks)
    t_att = time.perf_counter() - t0
    rows = rng.integers(0, N, CPU_SAMPLE_ROWS)
    log(f"[bench] cpu baseline: oracle dense attention of {len(rows)} rows")
    t0 = time.perf_counter()
    od, _ = O.dense_causal(qs, ks, vs, rows=rows, heads=[(0, 0)])
    t_dense = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    groups = spec.batch * spec.heads_kv
    nblk = spec.batch * spec.heads_q * nb
    nrows = spec.batch * spec.heads_q * N
    plan_ms = t_plan * groups * 1e3
    s2o_ms = (t_stop + t_att) / len(blocks) * nblk * 1e3
    dense_ms = t_dense / len(rows) * nrows * 1e3
    mask = ~np.isnan(o_ref[..., 0])
    err = float(np.abs(gpu["o"][mask] - o_ref[mask]).max())
    mse = float(np.mean((gpu["o"][mask] - o_ref[mask]) ** 2))
    derr = float(np.abs(gpu["o_dense"][0, 0, rows] - od[0, 0, rows]).max())
    ok_plan = (np.array_equal(gpu["pi_k"][0, 0], ref.pi_k[0, 0])
               and np.array_equal(gpu["pi_q"][0, :G], ref.pi_q[0])
               and np.array_equal(gpu["L"][0, 0], ref.L[0, 0]))
    stops_ok = all(n_gpu[b, h, I] == n_use[b, h, I] for b, h, I in blocks)
    return {"value": round(plan_ms + s2o_ms, 1), "unit": "ms/layer",
            "cores": cores, "blas_threads": blas, "kind": "oracle",
            "parts_ms": {"plan": round(plan_ms, 1),
                         "s2o_attention": round(s2o_ms, 1),
                         "dense_attention": round(dense_ms, 1)},
            "sample": f"oracle plan of 1 of {groups} KV groups "
                      f"({t_plan:.2f} s), stop points and attention of "
                      f"{len(blocks)} of {nblk} query blocks "
                      f"({(t_stop + t_att) * 1e3 / len(blocks):.1f} ms each), "
                      f"dense attention of {len(rows)} of {nrows} rows "
                      f"({t_dense * 1e3 / len(rows):.2f} ms each); each "
                      f"extrapolated linearly to the layer; value = plan + "
                      f"S2O attention",
            "extrapolated": True,
            "validation": {
                "plan_group0_bit_exact": bool(ok_plan),
                "sampled_blocks": len(blocks), "stop_ties": ties,
                "stop_points_equal": bool(stops_ok),
                "max_abs_err": err, "mse": mse,
                "dense_sampled_rows_max_abs_err": derr,
                "within_tolerance": bool(err <= 2e-2 and mse <= 1e-4
                                         and derr <= 2e-2 and ok_plan
                                         and stops_ok)}}


if __name__ == "__main__":
    main()
