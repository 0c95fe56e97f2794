"""The pins are strong enough: each planted mistake in a copy of the oracle
makes at least one pin fail (mistakes are planted on the CPU, in the copy
only; the real oracle is untouched)."""
import pathlib
import sys
import types

import pytest

import oracle.s2o as S2O
from tests import oracle_pins as P

SRC = pathlib.Path(S2O.__file__).read_text()

# (name, exact text in oracle/s2o.py, replacement)
MUTANTS = [
    ("sel_local_off_by_one", "local = i - (i // S) * S + 1",
     "local = i - (i // S) * S"),
    ("sel_far_natural_order", "far[pl.pi_q[b, h]] = per_row * BLOCK",
     "far[:] = per_row * BLOCK"),
    ("sel_far_one_key_per_tile", "far[pl.pi_q[b, h]] = per_row * BLOCK",
     "far[pl.pi_q[b, h]] = per_row"),
    ("density_denominator_x2", "/ (B * Hq * nb * (nb + 1) / 2),",
     "/ (B * Hq * nb * (nb + 1)),"),
    ("density_diag_strict", "diag_tiles += int((rows.max(axis=1) >= j0).sum())",
     "diag_tiles += int((rows.max(axis=1) > j0).sum())"),
    ("density_diag_first_row", "diag_tiles += int((rows.max(axis=1) >= j0).sum())",
     "diag_tiles += int((rows[:, 0] >= j0).sum())"),
    ("sparsity_pairs_n2", "total_pairs = B * Hq * N * (N + 1) / 2",
     "total_pairs = B * Hq * N * N / 2"),
    ("mse_abs", "out[\"mse\"] = float(np.mean((o - o_dense) ** 2))",
     "out[\"mse\"] = float(np.mean(np.abs(o - o_dense)))"),
    ("stop_after_next", "return int(below[0]), ps[:below[0] + 1]",
     "return int(below[0]) + 1, ps[:below[0] + 1]"),
    ("running_sum_from_zero", "run = np.cumsum(np.concatenate(([acc], E)))[:-1]",
     "run = np.cumsum(np.concatenate(([0.0], E)))[:-1]"),
    ("local_from_segment_start", "j0 = t * S + BLOCK * np.arange(S // BLOCK)",
     "j0 = BLOCK * np.arange(S // BLOCK)"),
    ("topk_tie_desc", "order = np.lexsort((np.arange(ntl), -r))   # r desc, position asc",
     "order = np.lexsort((-np.arange(ntl), -r))"),
    ("topk_ascending", "order = np.lexsort((np.arange(ntl), -r))   # r desc, position asc",
     "order = np.lexsort((np.arange(ntl), r))"),
    ("topk_natural_rows", "qs = qx_cache[(b, h)][rows].sum(axis=0)",
     "qs = qx_cache[(b, h)][I * BLOCK:(I + 1) * BLOCK].sum(axis=0)"),
    ("topk_first_key", "ks = kx_cache[(b, g)][tiles].sum(axis=1)",
     "ks = kx_cache[(b, g)][tiles[:, 0]]"),
    ("topk_one_more", "sel[order[:min(K, ntl)]] = True",
     "sel[order[:min(K + 1, ntl)]] = True"),
    ("topk_global_order", "sel[order[:min(K, ntl)]] = True",
     "sel[:min(K, ntl)] = True"),
    ("exact_mean_not_max", "mx = z.reshape(BLOCK, -1, BLOCK).max(axis=(0, 2))",
     "mx = z.reshape(BLOCK, -1, BLOCK).mean(axis=(0, 2))"),
    ("exact_strict", "sel = mx >= theta", "sel = mx > theta"),
    ("exact_no_kappa", "z = kap * (q[rows] @ k[tiles.reshape(-1)].T)        # 64 x (t S)",
     "z = (q[rows] @ k[tiles.reshape(-1)].T)"),
    ("attend_mask_ignored", "far = tiles[np.asarray(tile_mask[(b, h, I)], bool)].reshape(-1)",
     "far = tiles.reshape(-1)"),
    ("budget_off_by_one", "n_I[b, h, I] = min(budget, t * S // BLOCK)",
     "n_I[b, h, I] = min(budget + 1, t * S // BLOCK)"),
    ("budget_ignores_segment", "n_I[b, h, I] = min(budget, t * S // BLOCK)",
     "n_I[b, h, I] = budget"),
    ("segkv_tile_tie_desc", "Lt = tiles[np.lexsort((tid, -tscore))].reshape(-1)",
     "Lt = tiles[np.lexsort((-tid, -tscore))].reshape(-1)"),
    ("segkv_tiles_ascending", "Lt = tiles[np.lexsort((tid, -tscore))].reshape(-1)",
     "Lt = tiles[np.lexsort((tid, tscore))].reshape(-1)"),
    ("segkv_score_first_key", "tscore = v[tiles].sum(axis=1)",
     "tscore = v[tiles[:, 0]]"),
    ("segkv_keys_ascending", "seg[np.lexsort((seg, -v[seg]))]",
     "seg[np.lexsort((seg, v[seg]))]"),
    ("local_only_ignored", "    if pl.flags & SA_LOCAL_ONLY:\n", "    if False:\n"),
    ("recall_strict_causal", "causal = j[None, :] <= rows[:, None]",
     "causal = j[None, :] < rows[:, None]"),
    ("recall_no_far", "                sel |= mark[None, :]\n", "\n"),
    ("recall_segment_off_by_one", "sel = causal & (j[None, :] >= t * S)",
     "sel = causal & (j[None, :] > t * S)"),
    ("floor_not_rint", "y = np.rint(x * 256.0)", "y = np.floor(x * 256.0)"),
    ("scale_128", "y = np.rint(x * 256.0)", "y = np.rint(x * 128.0)"),
    ("clip_bounds", "np.clip(y, -32768.0, 32767.0)",
     "np.clip(y, -32767.0, 32767.0)"),
    ("kv_ascending", "order = np.lexsort((idx, -v))",
     "order = np.lexsort((idx, v))"),
    ("kv_tie_desc", "order = np.lexsort((idx, -v))",
     "order = np.lexsort((-idx, -v))"),
    ("q_ascending", "np.lexsort((seg, -u[seg]))]", "np.lexsort((seg, u[seg]))]"),
    ("drop_prefix", "(t * S) * top - BLOCK * prefix", "(t * S) * top"),
    ("swap_factors", "(t * S) * top - BLOCK * prefix",
     "BLOCK * top - (t * S) * prefix"),
    ("top_from_prefix", "top = kx[Lt[:BLOCK]].sum(axis=0)",
     "top = kx[:BLOCK].sum(axis=0)"),
    ("restrict_le", "Lt = order[order < t * S]",
     "Lt = order[order <= t * S][:t * S]"),
    ("stop_le", "below = np.flatnonzero(ps < tau)",
     "below = np.flatnonzero(ps <= tau)"),
    ("diag_weight", "acc += (nv[c] / BLOCK) * math.exp",
     "acc += nv[c] * math.exp"),
    ("tile_mass_1", "E = BLOCK * np.exp(kap * (tile_means @ qbar))",
     "E = np.exp(kap * (tile_means @ qbar))"),
    ("no_running_sum", "run = np.cumsum(np.concatenate(([acc], E)))[:-1]",
     "run = np.full(len(E), acc)"),
    ("estimate_no_kappa", "E = BLOCK * np.exp(kap * (tile_means @ qbar))",
     "E = BLOCK * np.exp(tile_means @ qbar)"),
    ("local_means_shifted", "local_means = block_means(k64, np.arange(t * S, (t + 1) * S))",
     "local_means = block_means(k64, np.arange(t * S - S, t * S))"),
    ("ratio_without_self", "ps = E / (run + E)", "ps = E / run"),
    ("qbar_natural_rows", "qbar = q64[rows].mean(axis=0)",
     "qbar = q64[I * BLOCK:(I + 1) * BLOCK].mean(axis=0)"),
    ("nvis_clip63", "np.clip(rows[None, :] - j0[:, None] + 1, 0, BLOCK)",
     "np.clip(rows[None, :] - j0[:, None], 0, BLOCK)"),
    ("dense_kappa_1_over_d", "return 1.0 / math.sqrt(d)", "return 1.0 / d"),
    ("dense_mask_ge", "z[np.arange(N)[None, :] > r[:, None]] = -np.inf",
     "z[np.arange(N)[None, :] >= r[:, None]] = -np.inf"),
    ("attend_mask_ge", "z[:, :S][local[None, :] > rows[:, None]] = -np.inf",
     "z[:, :S][local[None, :] >= rows[:, None]] = -np.inf"),
    ("attend_one_more_tile", "[:n * BLOCK] if t > 0", "[:(n + 1) * BLOCK] if t > 0"),
    ("attend_lse_no_max", "lse[b, h, rows] = (m + np.log(s))[:, 0]",
     "lse[b, h, rows] = np.log(s)[:, 0]"),
]


def load_mutant(name, old, new):
    assert SRC.count(old) == 1, f"{name}: anchor text not unique/present"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = f"<mutant {name}>"
    sys.modules[mod.__name__] = mod
    try:
        exec(compile(SRC.replace(old, new), mod.__file__, "exec"),
             mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = load_mutant(name, old, new)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"planted mistake '{name}' passed every pin"
