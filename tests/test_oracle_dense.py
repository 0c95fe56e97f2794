"""Pins of the oracle's dense causal attention (AB-Sparse page, Eq. (1)).

Pinned against: torch's float64 scaled-dot-product attention on the CPU (a
library routine), closed forms (identical keys, constant values, one
dominant key), and causality.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from tests.conftest import bits_of


def _rand_bits(rng, shape, scale=1.0):
    return bits_of(scale * rng.standard_normal(shape))


@pytest.mark.parametrize("Hq,Hkv,N,d", [(1, 1, 97, 16), (4, 2, 130, 64),
                                         (2, 1, 64, 128)])
def test_dense_matches_torch_sdpa_float64(rng, Hq, Hkv, N, d):
    q = _rand_bits(rng, (1, Hq, N, d), 2.0)
    k = _rand_bits(rng, (1, Hkv, N, d), 2.0)
    v = _rand_bits(rng, (1, Hkv, N, d))
    o, lse = O.dense_causal(q, k, v)
    G = Hq // Hkv
    tq = torch.from_numpy(O.decode_bf16(q))
    tk = torch.from_numpy(O.decode_bf16(k)).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(O.decode_bf16(v)).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_dense_identical_keys_is_prefix_mean(rng):
    # all keys equal: every visible key has the same logit, so row i is the
    # plain mean of v_0..v_i and lse_i = kappa q_i . k + log(i + 1)
    N, d = 80, 32
    q = _rand_bits(rng, (1, 1, N, d))
    k = np.broadcast_to(_rand_bits(rng, (1, 1, 1, d)), (1, 1, N, d)).copy()
    v = _rand_bits(rng, (1, 1, N, d))
    o, lse = O.dense_causal(q, k, v)
    v64 = O.decode_bf16(v)[0, 0]
    ref = np.cumsum(v64, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.abs(o[0, 0] - ref).max() < 1e-13
    z = O.decode_bf16(q)[0, 0] @ O.decode_bf16(k)[0, 0, 0] / math.sqrt(d)
    assert np.abs(lse[0, 0] - (z + np.log(np.arange(1, N + 1)))).max() < 1e-12


def test_dense_constant_values(rng):
    N, d = 50, 16
    q = _rand_bits(rng, (1, 1, N, d), 3.0)
    k = _rand_bits(rng, (1, 1, N, d), 3.0)
    row = _rand_bits(rng, (d,))
    v = np.broadcast_to(row, (1, 1, N, d)).copy()
    o, _ = O.dense_causal(q, k, v)
    assert np.abs(o[0, 0] - O.decode_bf16(row)[None]).max() < 1e-13


def test_dense_one_dominant_key(rng):
    # key 3 is aligned with every query and very large: rows i >= 3 return
    # v_3, rows i < 3 do not see it
    N, d = 40, 16
    qf = np.zeros((1, 1, N, d))
    qf[..., 0] = 1.0
    kf = 0.01 * rng.standard_normal((1, 1, N, d))
    kf[0, 0, 3, 0] = 400.0
    q, k = bits_of(qf), bits_of(kf)
    v = _rand_bits(rng, (1, 1, N, d))
    o, _ = O.dense_causal(q, k, v)
    v64 = O.decode_bf16(v)[0, 0]
    assert np.abs(o[0, 0, 3:] - v64[3][None]).max() < 1e-12
    assert np.abs(o[0, 0, 0] - v64[0]).max() < 1e-15


def test_dense_is_causal(rng):
    N, d = 64, 32
    q = _rand_bits(rng, (1, 1, N, d))
    k = _rand_bits(rng, (1, 1, N, d))
    v = _rand_bits(rng, (1, 1, N, d))
    o, _ = O.dense_causal(q, k, v)
    i = 20
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, i + 1:] = _rand_bits(rng, (N - i - 1, d))
    v2[0, 0, i + 1:] = _rand_bits(rng, (N - i - 1, d))
    o2, _ = O.dense_causal(q, k2, v2)
    assert np.array_equal(o[0, 0, :i + 1], o2[0, 0, :i + 1])
    assert not np.array_equal(o[0, 0, i + 1:], o2[0, 0, i + 1:])
