"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle (bit-exact indices, stop points up to
documented near-tau ties, outputs within the bf16 tolerance)."""
from __future__ import annotations

import sys

import numpy as np

# Output tolerance against the float64 oracle (bf16 inputs and output, fp32
# accumulation): max-abs and mean squared error.
MAX_ABS_TOL = 2e-2
MSE_TOL = 1e-4
LSE_TOL = 2e-3
# A stop decision is a near-tau tie when the oracle's ratio is within this
# relative distance of tau: the GPU evaluates a tile's mean logit in fp32
# (sum of the block's queries . sum of the tile's keys), the oracle in
# float64.
TIE_REL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda:0").view(torch.bfloat16)


def bf16_tensor_to_f64(t):
    import torch
    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def run_gpu(q, k, v, segment, tau, flags=0, kv_order=None, budget=None,
            max_theta=None, topk=None):
    import torch
    import permuted_block_sparse_amd as pbs
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    pl = pbs.plan(tq, tk, segment, tau, flags=flags)
    if budget is not None:
        pl.set_budget(budget)
    if max_theta is not None:
        pl.set_max_threshold(max_theta)
    if kv_order is not None:
        pl.set_kv_order(torch.from_numpy(
            np.ascontiguousarray(kv_order, dtype=np.int32)).to("cuda:0"))
    if topk is not None:
        pl.set_topk(topk)
    o, lse = pbs.prefill(pl, tq, tk, tv, return_lse=True)
    torch.cuda.synchronize()
    extra = {"topk_masks": pl.topk_masks()} if topk is not None else {}
    return {**extra,
        "o": bf16_tensor_to_f64(o), "lse": lse.cpu().numpy().astype(np.float64),
        "pi_k": pl.pi_k(), "pi_q": pl.pi_q(), "L": pl.restricted_lists(),
        "n_I": pl.n_I(), "key_score": pl.key_score(),
        "query_score": pl.query_score(), "contrast": pl.contrast(),
        "pooled": pl.pooled(), "plan": pl, "tensors": (tq, tk, tv, o),
    }


def assert_plan_equal(g, pl):
    """Indices and integer scores: bit-exact."""
    B, Hq, N = pl.pi_q.shape
    assert np.array_equal(g["pooled"], pl.pooled), "pooled query sums differ"
    assert np.array_equal(g["key_score"], pl.key_score), "key scores differ"
    assert np.array_equal(g["pi_k"], pl.pi_k), "global KV order differs"
    if pl.L.shape[-1]:
        assert np.array_equal(g["L"], pl.L), "restricted lists differ"
    assert np.array_equal(g["contrast"], pl.contrast), "contrast differs"
    assert np.array_equal(g["query_score"], pl.query_score), "u differs"
    assert np.array_equal(g["pi_q"], pl.pi_q), "query order differs"


def stop_mismatches(n_gpu, n_orc, traces, tau, blocks=None):
    """Blocks whose stop points differ; each must be a documented near-tau
    tie: the oracle's ratio at the first differing decision is within
    TIE_REL * tau of tau."""
    diff = np.argwhere(n_gpu != n_orc)
    out = []
    for b, h, I in diff:
        if n_orc[b, h, I] < 0:
            continue
        m = int(min(n_gpu[b, h, I], n_orc[b, h, I]))
        p = traces[(int(b), int(h), int(I))][m]
        assert abs(p - tau) <= TIE_REL * tau, (
            f"stop point differs at block {(b, h, I)}: gpu {n_gpu[b, h, I]}"
            f" oracle {n_orc[b, h, I]}, ratio {p!r} vs tau {tau!r}")
        out.append((int(b), int(h), int(I)))
    return out


def rows_of_blocks(pi_q, blocks):
    return [(b, h, pi_q[b, h, 64 * I:64 * I + 64]) for b, h, I in blocks]


def assert_outputs_close(o_gpu, o_ref, lse_gpu=None, lse_ref=None, mask=None):
    if mask is None:
        mask = ~np.isnan(o_ref[..., 0])
    a, r = o_gpu[mask], o_ref[mask]
    err = np.abs(a - r)
    mse = float(np.mean((a - r) ** 2))
    assert err.max() <= MAX_ABS_TOL, f"max abs err {err.max()}"
    assert mse <= MSE_TOL, f"mse {mse}"
    if lse_gpu is not None:
        le = np.abs(lse_gpu[mask] - lse_ref[mask]).max()
        assert le <= LSE_TOL, f"lse err {le}"
    return float(err.max()), mse


def unpack_tile_mask(words, ntl):
    """Bitmask words (uint32, bit p of word w = position 32 w + p) -> bool
    per position; also asserts that no bit past ntl is set."""
    bits = np.unpackbits(np.ascontiguousarray(words).view(np.uint8),
                         bitorder="little").astype(bool)
    assert not bits[ntl:].any(), "bits set past the end of L_t"
    return bits[:ntl]
