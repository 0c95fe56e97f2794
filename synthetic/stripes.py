"""Stripe-structured synthetic Q/K/V (bfloat16 bit patterns), seeded.

The S2O summary page ("S2O: Early Stopping for Sparse Attention via Online
Permutation", Summary) describes real attention maps as thin vertical,
horizontal and diagonal stripes. No model weights or long-context datasets
are available here, so these tensors stand in for the Llama-3.1-8B and
Qwen3-8B layers that page measures. The recipe plants the three stripe
kinds on top of i.i.d. N(0, 1) noise:

* vertical stripes: for every query head h, a unit direction u_h and a set
  of key positions; those keys get ``vert_gain * u_h`` and every query of
  head h gets ``query_gain * u_h``, so the chosen keys draw extra attention
  from every query of that head;
* a diagonal local band: positions are cut into consecutive windows of
  ``window`` tokens; every (KV head, window) pair gets its own unit
  direction r, added as ``window_gain * r`` to the keys and to the queries
  of that window (queries and keys of one window then attend to each other);
* horizontal stripes: a set of query positions per head whose rows are
  multiplied by ``horiz_factor`` (applied last), giving those queries
  sharper attention rows.

Draw order (fixed; every consumer regenerates the same tensors from the
seed): Q, K, V base draws; the per-head vertical counts when a range is
given; then per batch element: per query head (u_h, key positions), per KV
head the window directions, per query head the horizontal positions.

Everything is drawn in float32 and rounded once to bfloat16 with
round-to-nearest-even. Values are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class StripeSpec:
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int = 128
    n_vert: int = 0                    # vertical-stripe keys per query head
    n_vert_range: Optional[Tuple[int, int]] = None  # per-head Uniform{lo..hi}
    n_horiz: int = 0                   # horizontal-stripe queries per head
    window: int = 0                    # local band width (0 = none)
    vert_gain: float = 3.0
    query_gain: float = 1.0
    window_gain: float = 2.0
    horiz_factor: float = 2.0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _unit(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / n


def make_stripe_inputs(spec: StripeSpec):
    """Return (q, k, v) as uint16 bfloat16 bit arrays.

    Shapes: q [B, Hq, N, d]; k, v [B, Hkv, N, d]; all C-contiguous.
    """
    B, Hq, Hkv, N, d = (spec.batch, spec.heads_q, spec.heads_kv,
                        spec.seq_len, spec.head_dim)
    if Hq % Hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if spec.n_vert_range is not None:
        lo, hi = spec.n_vert_range
        n_vert = rng.integers(lo, hi + 1, size=(B, Hq))
    else:
        n_vert = np.full((B, Hq), spec.n_vert, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            u = _unit(rng, (d,))
            nv = int(n_vert[b, h])
            if nv > 0:
                pos = rng.choice(N, nv, replace=False)
                k[b, g, pos] += np.float32(spec.vert_gain) * u
            q[b, h] += np.float32(spec.query_gain) * u
        if spec.window > 0:
            n_win = -(-N // spec.window)
            for g in range(Hkv):
                r = _unit(rng, (n_win, d))
                band = np.repeat(r, spec.window, axis=0)[:N]
                band *= np.float32(spec.window_gain)
                k[b, g] += band
                q[b, g * G:(g + 1) * G] += band
        for h in range(Hq):
            if spec.n_horiz > 0:
                pos = rng.choice(N, spec.n_horiz, replace=False)
                q[b, h, pos] *= np.float32(spec.horiz_factor)
    out = []
    for x in (q, k, v):
        bits = np.empty(x.shape, dtype=np.uint16)
        for b in range(x.shape[0]):
            for h in range(x.shape[1]):
                bits[b, h] = round_to_bf16_bits(x[b, h])
        out.append(bits)
    return tuple(out)
