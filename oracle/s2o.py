"""Plain CPU reference of permuted, early-stopping block-sparse prefill attention.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Sources. "S2O summary" is the page "S2O: Early Stopping for Sparse Attention
via Online Permutation" (Elamur Research summary); "PBS-Attn page" is the
poster page "Sparser Block-Sparse Attention via Token Permutation";
"AB-Sparse page" is "AB-Sparse: Sparse Attention with Adaptive Block Size
for Accurate and Efficient Long-Context Inference".

Notation. b batch, h query head, g = h // G its KV head (G = Hq / Hkv), N
tokens, d head dim, S segment length, T = N / S segments, seg(i) = i // S,
blocks of 64 rows/keys, kappa = 1 / sqrt(d). Q is [B, Hq, N, d], K and V are
[B, Hkv, N, d], all given as bfloat16 bit patterns.

The pages describe the method in prose only (S2O summary, Summary, second
paragraph). Every point they leave open is fixed below and marked READING;
the same readings are used by the GPU path.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

SA_NO_QPERM = 1        # identity query order
SA_NO_KVPERM = 2       # identity key/value order
SA_NO_EARLYSTOP = 4    # never stop (same as tau = 0)
SA_LOCAL_ONLY = 8      # dense local window only: n_I = 0 for every block
SA_SEGMENT_KV = 16     # segment-local key order, tiles visited by tile score

BLOCK = 64


# --------------------------------------------------------------------------
# Inputs
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def kappa_of(d: int) -> float:
    """Softmax scale 1/sqrt(d) (AB-Sparse page, Eq. (1))."""
    return 1.0 / math.sqrt(d)


def fixed_point(bits: np.ndarray) -> np.ndarray:
    """Fixed-point image used for every ranking score (int64).

    READING: the pages say the orders are "ranked by stripe-level mean
    pooling" (S2O summary, Summary) and give no precision; the AB-Sparse page
    notes that pooled block centroids serve only for ranking and tolerate low
    precision (its centroid-quantisation discussion). Ranking is therefore
    done on exact integers so that any implementation reproduces the orders
    bit for bit: fx(x) = clamp(round_half_even(256 x), -32768, 32767).
    """
    x = decode_bf16(bits)
    y = np.rint(x * 256.0)                      # rint: round half to even
    y = np.clip(y, -32768.0, 32767.0)
    return y.astype(np.int64)


# --------------------------------------------------------------------------
# Dense causal attention
# --------------------------------------------------------------------------

def dense_causal(q_bits, k_bits, v_bits, rows: Optional[Sequence[int]] = None,
                 heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Causal softmax attention, AB-Sparse page Eq. (1), in float64.

    o_i = sum_{j <= i} softmax_j(kappa q_i . k_j) v_j, and
    lse_i = log sum_{j <= i} exp(kappa q_i . k_j).
    Returns (o [B, Hq, N, d], lse [B, Hq, N]); with ``rows`` only those rows
    are filled (others are NaN); ``heads`` limits the (b, h) pairs computed.
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // k_bits.shape[1]
    kap = kappa_of(d)
    o = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = heads if heads is not None else [(b, h) for b in range(B)
                                              for h in range(Hq)]
    for b, h in pairs:
        q = decode_bf16(q_bits[b, h])
        k = decode_bf16(k_bits[b, h // G])
        v = decode_bf16(v_bits[b, h // G])
        for c0 in range(0, len(rows), 256):
            r = rows[c0:c0 + 256]
            z = kap * (q[r] @ k.T)                       # [rows, N]
            z[np.arange(N)[None, :] > r[:, None]] = -np.inf
            m = z.max(axis=1, keepdims=True)
            p = np.exp(z - m)
            s = p.sum(axis=1, keepdims=True)
            o[b, h, r] = (p @ v) / s
            lse[b, h, r] = (m + np.log(s))[:, 0]
    return o, lse


# --------------------------------------------------------------------------
# The plan: both orders and the restricted key lists (integers only)
# --------------------------------------------------------------------------

@dataclass
class Plan:
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    segment: int
    flags: int
    pooled: np.ndarray        # P [B, Hkv, d] int64 (group query sum)
    key_score: np.ndarray     # v [B, Hkv, N] int64
    pi_k: np.ndarray          # [B, Hkv, N] global key/value order
    contrast: np.ndarray      # C [B, Hkv, T, d] int64 (row 0 unused, zero)
    query_score: np.ndarray   # u [B, Hq, N] int64
    pi_q: np.ndarray          # [B, Hq, N] segment-local query order
    L: np.ndarray             # [B, Hkv, S*T*(T-1)/2] restricted lists, t = 1..T-1

    @property
    def n_segments(self) -> int:
        return self.seq_len // self.segment

    @property
    def n_blocks(self) -> int:
        return self.seq_len // BLOCK


def list_offset(segment: int, t: int) -> int:
    """Start of L_t in the concatenation L_1, L_2, ... (|L_t| = t S)."""
    return segment * t * (t - 1) // 2


def restricted_list(pl: Plan, b: int, g: int, t: int) -> np.ndarray:
    o = list_offset(pl.segment, t)
    return pl.L[b, g, o:o + t * pl.segment]


def _check_shape(q_bits, k_bits, segment, block):
    B, Hq, N, d = q_bits.shape
    Bk, Hkv, Nk, dk = k_bits.shape
    if (Bk, Nk, dk) != (B, N, d) or Hq % Hkv:
        raise ValueError("Q/K shapes do not agree")
    if block != BLOCK:
        raise ValueError("block must be 64")
    if segment <= 0 or segment % block or N % segment:
        raise ValueError("need segment % 64 == 0 and seq_len % segment == 0")
    if N > (1 << 17):
        raise ValueError("seq_len above 2^17 overflows the int64 scores")
    return B, Hq, Hkv, N, d


def plan(q_bits, k_bits, segment: int, block: int = BLOCK,
         flags: int = 0, kv_order: Optional[np.ndarray] = None) -> Plan:
    """Build both orders and the restricted key lists (S2O summary, Summary).

    The page says S2O builds "lightweight index arrays": a segment-local
    query ordering and a global key/value ordering ranked by stripe-level
    mean pooling, and moves no tensor. Steps, per (b, KV head g):

    1. Pooled query: P = sum over the G query heads of g and all N rows of
       fx(q). READING: the global order pools all queries of the group (a
       mean up to the positive factor G N, which does not change ranks).
    2. Key stripe score: v_j = P . fx(k_j). A vertical stripe is one key
       column; by linearity P . k_j / (G N) is the mean of that column's
       logits over the pooled queries (mean pooling of the stripe).
    3. Global key/value order pi_K: keys by v descending, ties by smaller
       index first (READING: ties are not discussed on the pages).
    4. Causal restriction: for t >= 1, L_t = pi_K with every key j >= t S
       removed, order kept (|L_t| = t S). Segment t's queries only ever see
       tiles of L_t, so no query sees a future key. READING: the pages give a
       global order but do not say how causality is kept.
    5. Contrast vector: C_t = t S * sum_{j in L_t[0:64]} fx(k_j)
       - 64 * sum_{j < t S} fx(k_j), i.e. 64 t S times (mean of the top tile
       - mean of the whole visible prefix).
    6. Query stripe score: u_i = fx(q_i) . C_seg(i) for seg(i) >= 1, and 0 in
       segment 0. READING: the pages name the segment-local query ordering
       (S2O summary, Summary) and report that it raises sparsity (Key points,
       component ablation) but give no criterion; u_i measures how strongly
       query i prefers the most important keys over the average visible key.
    7. Segment-local query order pi_Q: inside each segment [t S, t S + S),
       queries by u descending, ties by smaller index. Query block I holds
       the original rows pi_Q[64 I : 64 I + 64], all inside one segment.

    Flags: SA_NO_KVPERM makes pi_K the identity, SA_NO_QPERM makes pi_Q the
    identity (the other steps are unchanged). ``kv_order`` ([B, Hkv, N])
    replaces pi_K by a given permutation (a test hook: with tau = 0 the
    output must not depend on it).

    SA_SEGMENT_KV replaces steps 3 and 4 by the segment-local key order of
    the PBS-Attn page (tokens permuted inside causal segments, abstract):
    pi_K sorts the keys of each segment [u S, u S + S) by v descending, ties
    by index; its 64-key chunks are the tiles (S is a multiple of 64, so no
    tile crosses a segment); L_t lists the tiles of segments 0 .. t - 1 by
    tile score (sum of v over the tile) descending, ties by tile index.
    READING: the PBS-Attn page gives the permutation inside segments but no
    visiting order; most-to-least-important visiting (S2O summary, Summary)
    needs one, and the tile score is the mean-pooled stripe score of the
    tile up to the factor 64. SA_NO_KVPERM takes precedence; ``kv_order``
    cannot be combined with it.
    """
    B, Hq, Hkv, N, d = _check_shape(q_bits, k_bits, segment, block)
    G = Hq // Hkv
    S = segment
    T = N // S
    pooled = np.zeros((B, Hkv, d), dtype=np.int64)
    key_score = np.zeros((B, Hkv, N), dtype=np.int64)
    pi_k = np.zeros((B, Hkv, N), dtype=np.int64)
    contrast = np.zeros((B, Hkv, T, d), dtype=np.int64)
    query_score = np.zeros((B, Hq, N), dtype=np.int64)
    pi_q = np.zeros((B, Hq, N), dtype=np.int64)
    L = np.zeros((B, Hkv, list_offset(S, T)), dtype=np.int64)
    idx = np.arange(N, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            # 1. pooled query of the group
            P = np.zeros(d, dtype=np.int64)
            for h in heads:
                P += fixed_point(q_bits[b, h]).sum(axis=0)
            pooled[b, g] = P
            # 2. key stripe scores (exact int64 dot products)
            kx = fixed_point(k_bits[b, g])
            v = kx @ P
            key_score[b, g] = v
            # 3. global order: v descending, then index ascending
            segment_kv = bool(flags & SA_SEGMENT_KV) and not (
                flags & SA_NO_KVPERM)
            if kv_order is not None:
                if segment_kv:
                    raise ValueError("kv_order with SA_SEGMENT_KV")
                order = np.asarray(kv_order[b, g], dtype=np.int64)
                assert np.array_equal(np.sort(order), idx)
            elif flags & SA_NO_KVPERM:
                order = idx.copy()
            elif segment_kv:
                order = np.concatenate([
                    seg[np.lexsort((seg, -v[seg]))]
                    for seg in (idx[u * S:(u + 1) * S] for u in range(T))])
            else:
                order = np.lexsort((idx, -v))
            pi_k[b, g] = order
            # 4. causal restriction (or the tile order of the segment-local
            # variant), 5. contrast vectors
            for t in range(1, T):
                if segment_kv:
                    tiles = order[:t * S].reshape(-1, BLOCK)
                    tscore = v[tiles].sum(axis=1)
                    tid = np.arange(len(tiles))
                    Lt = tiles[np.lexsort((tid, -tscore))].reshape(-1)
                else:
                    Lt = order[order < t * S]
                assert len(Lt) == t * S
                o = list_offset(S, t)
                L[b, g, o:o + t * S] = Lt
                top = kx[Lt[:BLOCK]].sum(axis=0)
                prefix = kx[:t * S].sum(axis=0)
                contrast[b, g, t] = (t * S) * top - BLOCK * prefix
            # 6. query stripe scores, 7. segment-local query order
            for h in heads:
                qx = fixed_point(q_bits[b, h])
                u = np.zeros(N, dtype=np.int64)
                for t in range(1, T):
                    rows = slice(t * S, (t + 1) * S)
                    u[rows] = qx[rows] @ contrast[b, g, t]
                query_score[b, h] = u
                if flags & SA_NO_QPERM:
                    pi_q[b, h] = idx
                else:
                    for t in range(T):
                        seg = idx[t * S:(t + 1) * S]
                        pi_q[b, h, t * S:(t + 1) * S] = seg[
                            np.lexsort((seg, -u[seg]))]
    return Plan(B, Hq, Hkv, N, d, S, flags, pooled, key_score, pi_k,
                contrast, query_score, pi_q, L)


# --------------------------------------------------------------------------
# Stop points (mean-pooled block estimates and the tau test)
# --------------------------------------------------------------------------

def block_means(k64: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Mean key of every consecutive 64-key tile of ``keys`` (float64)."""
    return k64[keys].reshape(len(keys) // BLOCK, BLOCK, -1).mean(axis=1)


def block_stop(qbar: np.ndarray, rows: np.ndarray, t: int,
               local_means: np.ndarray, tile_means: Optional[np.ndarray],
               S: int, tau: float, kap: float):
    """Stop point n_I of one query block and the ratios it was decided on.

    S2O summary, Summary: blocks are processed from most to least important
    and computation stops once a block's score falls under tau.

    READINGS (the page gives no formula):
      * block estimate: the mean-pooled logit of a 64 x 64 tile,
        s = kappa * qbar_I . kbar_tile (= the mean of the tile's 4096
        logits), and its estimated mass per query row E = n * exp(s), with
        n the average number of keys a row sees in that tile (64 for a
        sparse tile, n_vis / 64 for a diagonal block);
      * the dense local window is the query's own segment, computed exactly
        (S2O summary, Key points, component ablation); its estimated mass
        E_diag = sum_c (n_vis(I, c) / 64) exp(s_c) over its 64-key blocks c
        in ascending order starts the running total;
      * score normalisation: tile k's score is its share of the estimated
        mass seen so far including itself, p_k = E_k / (Acc_k + E_k) with
        Acc_0 = E_diag and Acc_{k+1} = Acc_k + E_k;
      * stop at the first k with p_k < tau (strict); n_I = that k, or all
        t S / 64 tiles when none fails. tau = 0 never stops.
    ``local_means`` holds the mean key of the segment's 64-key blocks,
    ``tile_means`` the mean key of the tiles of L_t in visiting order.
    Returns (n_I, p) where p holds p_0 .. p_{min(n_I, n_tiles - 1)}.
    """
    if t == 0:
        return 0, np.zeros(0)
    # dense local window estimate, blocks in ascending order; nv[c] = number
    # of (row, key) pairs of the block with key j0 + c' <= row, c' in 0..63
    j0 = t * S + BLOCK * np.arange(S // BLOCK)
    nv = np.clip(rows[None, :] - j0[:, None] + 1, 0, BLOCK).sum(axis=1)
    s_loc = kap * (local_means @ qbar)
    acc = 0.0
    for c in range(S // BLOCK):
        if nv[c] > 0:
            acc += (nv[c] / BLOCK) * math.exp(s_loc[c])
    # estimates past the stop point are computed but never used
    E = BLOCK * np.exp(kap * (tile_means @ qbar))
    # running total before tile k: E_diag + E_0 + ... + E_{k-1}, added in
    # that order (a cumulative sum adds left to right)
    run = np.cumsum(np.concatenate(([acc], E)))[:-1]
    ps = E / (run + E)
    below = np.flatnonzero(ps < tau)
    if len(below):
        return int(below[0]), ps[:below[0] + 1]
    return len(tile_means), ps


def stop_points(q_bits, k_bits, pl: Plan, tau: float,
                blocks: Optional[Sequence[Tuple[int, int, int]]] = None,
                budget: Optional[int] = None):
    """n_I for every query block (or the listed (b, h, I) blocks).

    Returns (n_I [B, Hq, N/64] int64 with -1 for blocks not computed,
    traces dict (b, h, I) -> array of p_k).

    SA_LOCAL_ONLY: no tile of L_t is visited (n_I = 0, empty traces) -- the
    "dense local window only" baseline of the S2O page's component ablation
    (Key points).

    ``budget`` >= 0: a fixed tile budget replaces the stop test; every block
    of segment t visits the first min(budget, t S / 64) tiles of L_t (the
    most important tiles of the mean-pooled ranking, the same count for
    every block -- the fixed-budget selection the S2O page's adaptive stop
    is compared with, Key points). SA_LOCAL_ONLY takes precedence.
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // pl.heads_kv
    S = pl.segment
    kap = kappa_of(d)
    if pl.flags & SA_NO_EARLYSTOP:
        tau = 0.0
    nb = N // BLOCK
    n_I = np.full((B, Hq, nb), -1, dtype=np.int64)
    traces = {}
    if blocks is None:
        blocks = [(b, h, I) for b in range(B) for h in range(Hq)
                  for I in range(nb)]
    if pl.flags & SA_LOCAL_ONLY:
        for b, h, I in blocks:
            n_I[b, h, I] = 0
            traces[(b, h, I)] = np.zeros(0)
        return n_I, traces
    if budget is not None and budget >= 0:
        for b, h, I in blocks:
            t = (I * BLOCK) // S
            n_I[b, h, I] = min(budget, t * S // BLOCK)
            traces[(b, h, I)] = np.zeros(0)
        return n_I, traces
    by_group: Dict[Tuple[int, int, int], list] = {}
    for b, h, I in blocks:
        by_group.setdefault((b, h // G, (I * BLOCK) // S), []).append((h, I))
    # decoded inputs of the current (b, KV head) only (groups are visited
    # in (b, g, t) order)
    cache: Dict[Tuple[int, int], tuple] = {}
    for (b, g, t), items in sorted(by_group.items()):
        if (b, g) not in cache:
            cache.clear()
            cache[(b, g)] = (decode_bf16(k_bits[b, g]), {})
        k64, q_heads = cache[(b, g)]
        local_means = block_means(k64, np.arange(t * S, (t + 1) * S))
        tile_means = (block_means(k64, restricted_list(pl, b, g, t))
                      if t > 0 else None)
        for h, I in items:
            if h not in q_heads:
                q_heads[h] = decode_bf16(q_bits[b, h])
            q64 = q_heads[h]
            rows = pl.pi_q[b, h, I * BLOCK:(I + 1) * BLOCK]
            qbar = q64[rows].mean(axis=0)
            n, ps = block_stop(qbar, rows, t, local_means, tile_means, S,
                               tau, kap)
            n_I[b, h, I] = n
            traces[(b, h, I)] = ps
    return n_I, traces


# --------------------------------------------------------------------------
# Attention over the selected set
# --------------------------------------------------------------------------

def attend(q_bits, k_bits, v_bits, pl: Plan, n_I: np.ndarray,
           blocks: Optional[Sequence[Tuple[int, int, int]]] = None,
           tile_mask: Optional[Dict[Tuple[int, int, int], np.ndarray]] = None):
    """Softmax attention of each query over its selected key set, float64.

    For query block I in segment t with stop point n_I, row i attends to
    Sel(i) = {j : seg(j) = t, j <= i} (the dense local window, causal) plus
    every key of the tiles L_t[0 : 64 n_I]; the softmax is renormalised over
    Sel(i) and skipped keys contribute nothing (block-sparse attention as on
    the PBS-Attn page; scale as in AB-Sparse Eq. (1)). The result is written
    back to the query's original row: no tensor is moved (S2O summary,
    Summary). Returns (o [B, Hq, N, d], lse [B, Hq, N]) with NaN in rows of
    blocks not computed. ``tile_mask`` ((b, h, I) -> bool per tile of L_t)
    selects an arbitrary subset of the tiles instead of the first n_I (the
    exact per-block max test).
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // pl.heads_kv
    S = pl.segment
    kap = kappa_of(d)
    o = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    nb = N // BLOCK
    if blocks is None:
        blocks = [(b, h, I) for b in range(B) for h in range(Hq)
                  for I in range(nb)]
    by_head: Dict[Tuple[int, int], list] = {}
    for b, h, I in blocks:
        by_head.setdefault((b, h), []).append(I)
    for (b, h), Is in sorted(by_head.items()):
        g = h // G
        q = decode_bf16(q_bits[b, h])
        k = decode_bf16(k_bits[b, g])
        v = decode_bf16(v_bits[b, g])
        for I in Is:
            rows = pl.pi_q[b, h, I * BLOCK:(I + 1) * BLOCK]
            t = (I * BLOCK) // S
            local = np.arange(t * S, (t + 1) * S)
            n = int(n_I[b, h, I])
            if tile_mask is not None and t > 0:
                tiles = restricted_list(pl, b, g, t).reshape(-1, BLOCK)
                far = tiles[np.asarray(tile_mask[(b, h, I)], bool)].reshape(-1)
            else:
                far = (restricted_list(pl, b, g, t)[:n * BLOCK] if t > 0
                       else np.zeros(0, dtype=np.int64))
            keys = np.concatenate([local, far])
            z = kap * (q[rows] @ k[keys].T)
            z[:, :S][local[None, :] > rows[:, None]] = -np.inf
            m = z.max(axis=1, keepdims=True)
            p = np.exp(z - m)
            s = p.sum(axis=1, keepdims=True)
            o[b, h, rows] = (p @ v[keys]) / s
            lse[b, h, rows] = (m + np.log(s))[:, 0]
    return o, lse


def exact_max_selection(q_bits, k_bits, pl: Plan, theta: float,
                        blocks: Optional[Sequence[Tuple[int, int, int]]] = None):
    """The exact per-block maximum test of the BSFA page (abstract): every
    tile of L_t is scored exactly and attended only if the largest scaled
    logit of the 64 x 64 tile, max over its query rows i and keys j of
    kappa q_i . k_j, is at least theta (a given threshold; the page
    calibrates one per layer and head on data). READING: no early stop in
    this mode, the dense local window is always attended, and an absolute
    threshold makes the selection independent of the visiting order.
    Returns (counts n_I [B, Hq, N/64], masks (b, h, I) -> bool per tile,
    maxima (b, h, I) -> tile maxima).
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // pl.heads_kv
    S = pl.segment
    kap = kappa_of(d)
    nb = N // BLOCK
    n_I = np.full((B, Hq, nb), -1, dtype=np.int64)
    masks, maxima = {}, {}
    if blocks is None:
        blocks = [(b, h, I) for b in range(B) for h in range(Hq)
                  for I in range(nb)]
    for b, h, I in blocks:
        g = h // G
        t = (I * BLOCK) // S
        if t == 0 or pl.flags & SA_LOCAL_ONLY:
            n_I[b, h, I] = 0
            masks[(b, h, I)] = np.zeros(t * S // BLOCK, dtype=bool)
            maxima[(b, h, I)] = np.zeros(0)
            continue
        q = decode_bf16(q_bits[b, h])
        k = decode_bf16(k_bits[b, g])
        rows = pl.pi_q[b, h, I * BLOCK:(I + 1) * BLOCK]
        tiles = restricted_list(pl, b, g, t).reshape(-1, BLOCK)
        z = kap * (q[rows] @ k[tiles.reshape(-1)].T)        # 64 x (t S)
        mx = z.reshape(BLOCK, -1, BLOCK).max(axis=(0, 2))
        sel = mx >= theta
        n_I[b, h, I] = int(sel.sum())
        masks[(b, h, I)] = sel
        maxima[(b, h, I)] = mx
    return n_I, masks, maxima


def topk_selection(q_bits, k_bits, pl: Plan, K: int,
                            blocks: Optional[Sequence[Tuple[int, int, int]]]
                            = None):
    """Per-block Top-K tile selection from mean-pooled centroids, instead of
    the tau stop: the AB-Sparse page's block-sparse workflow (the paragraph
    around its Figure 2 and the footnote on mean pooling) scores every key
    block by the product of the query with the block's centroid, the mean
    of its keys, and attends the K best blocks. Here the query side is the
    query block's mean query as well (one selection per 64-row block, as
    the attention works on 64 x 64 tiles).

    For query block I of segment t: every tile T_k of L_t gets the score
    r_k = (sum of fx(q_i) over the block's 64 rows) . (sum of fx(k_j) over
    the tile's 64 keys) -- 4096 times the block's mean query against the
    tile's centroid, both in the fixed-point images of the orders; the
    block attends to the min(K, t S / 64) tiles of highest r_k, ties by
    smaller position in L_t. READING: the page ranks by real-valued
    products; as for every order of this method, the ranking is done on
    exact integers (fixed-point images, int64 sums) so that it is
    reproducible bit for bit; the dense local window is always attended;
    SA_LOCAL_ONLY still attends to no tile.
    Returns (counts n_I [B, Hq, N/64], masks (b, h, I) -> bool per tile of
    L_t, scores (b, h, I) -> int64 r per tile).
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // pl.heads_kv
    S = pl.segment
    nb = N // BLOCK
    n_I = np.full((B, Hq, nb), -1, dtype=np.int64)
    masks, scores = {}, {}
    if blocks is None:
        blocks = [(b, h, I) for b in range(B) for h in range(Hq)
                  for I in range(nb)]
    kx_cache: Dict[Tuple[int, int], np.ndarray] = {}
    qx_cache: Dict[Tuple[int, int], np.ndarray] = {}
    for b, h, I in blocks:
        g = h // G
        t = (I * BLOCK) // S
        ntl = t * S // BLOCK
        if t == 0 or pl.flags & SA_LOCAL_ONLY or K <= 0:
            n_I[b, h, I] = 0
            masks[(b, h, I)] = np.zeros(ntl, dtype=bool)
            scores[(b, h, I)] = np.zeros(0, dtype=np.int64)
            continue
        if (b, g) not in kx_cache:
            kx_cache[(b, g)] = fixed_point(k_bits[b, g])
        if (b, h) not in qx_cache:
            qx_cache[(b, h)] = fixed_point(q_bits[b, h])
        rows = pl.pi_q[b, h, I * BLOCK:(I + 1) * BLOCK]
        qs = qx_cache[(b, h)][rows].sum(axis=0)                  # int64 [d]
        tiles = restricted_list(pl, b, g, t).reshape(-1, BLOCK)
        ks = kx_cache[(b, g)][tiles].sum(axis=1)                 # int64 [ntl, d]
        r = ks @ qs                                              # int64 [ntl]
        order = np.lexsort((np.arange(ntl), -r))   # r desc, position asc
        sel = np.zeros(ntl, dtype=bool)
        sel[order[:min(K, ntl)]] = True
        n_I[b, h, I] = int(sel.sum())
        masks[(b, h, I)] = sel
        scores[(b, h, I)] = r
    return n_I, masks, scores


def recall(q_bits, k_bits, pl: Plan, n_I: np.ndarray,
           blocks: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Attention recall of each row: the share of its dense causal attention
    mass (softmax of AB-Sparse Eq. (1) over every key j <= i) that falls on
    its selected set Sel(i) (own-segment keys j <= i plus the first n_I
    tiles of L_t). 1 when nothing is skipped; float64, [B, Hq, N], NaN in
    rows of blocks not listed.
    """
    B, Hq, N, d = q_bits.shape
    G = Hq // pl.heads_kv
    S = pl.segment
    kap = kappa_of(d)
    r = np.full((B, Hq, N), np.nan)
    nb = N // BLOCK
    if blocks is None:
        blocks = [(b, h, I) for b in range(B) for h in range(Hq)
                  for I in range(nb)]
    by_head: Dict[Tuple[int, int], list] = {}
    for b, h, I in blocks:
        by_head.setdefault((b, h), []).append(I)
    for (b, h), Is in sorted(by_head.items()):
        g = h // G
        q = decode_bf16(q_bits[b, h])
        k = decode_bf16(k_bits[b, g])
        for I in Is:
            rows = pl.pi_q[b, h, I * BLOCK:(I + 1) * BLOCK]
            t = (I * BLOCK) // S
            top = int(rows.max()) + 1
            z = kap * (q[rows] @ k[:top].T)
            j = np.arange(top)
            causal = j[None, :] <= rows[:, None]
            z[~causal] = -np.inf
            w = np.exp(z - z.max(axis=1, keepdims=True))
            sel = causal & (j[None, :] >= t * S)      # own segment, j <= i
            n = int(n_I[b, h, I])
            if t > 0 and n > 0:
                far = restricted_list(pl, b, g, t)[:n * BLOCK]
                mark = np.zeros(top, dtype=bool)
                mark[far[far < top]] = True
                sel |= mark[None, :]
            r[b, h, rows] = (w * sel).sum(axis=1) / w.sum(axis=1)
    return r


def s2o_attention(q_bits, k_bits, v_bits, segment: int, tau: float,
                  flags: int = 0, block: int = BLOCK):
    """Whole method on every block: plan, stop points, attention."""
    pl = plan(q_bits, k_bits, segment, block, flags)
    n_I, traces = stop_points(q_bits, k_bits, pl, tau)
    o, lse = attend(q_bits, k_bits, v_bits, pl, n_I)
    return o, lse, pl, n_I, traces


# --------------------------------------------------------------------------
# Metrics
# --------------------------------------------------------------------------

def selected_counts(pl: Plan, n_I: np.ndarray) -> np.ndarray:
    """|Sel(i)| for every row (original order), int64 [B, Hq, N]."""
    B, Hq, N = pl.batch, pl.heads_q, pl.seq_len
    S = pl.segment
    cnt = np.zeros((B, Hq, N), dtype=np.int64)
    i = np.arange(N)
    local = i - (i // S) * S + 1
    for b in range(B):
        for h in range(Hq):
            per_row = np.repeat(n_I[b, h], BLOCK)     # in permuted order
            far = np.zeros(N, dtype=np.int64)
            far[pl.pi_q[b, h]] = per_row * BLOCK
            cnt[b, h] = local + far
    return cnt


def metrics(pl: Plan, n_I: np.ndarray, o: Optional[np.ndarray] = None,
            o_dense: Optional[np.ndarray] = None) -> dict:
    """Sparsity, tile density and MSE (S2O summary, Key points).

    * pair sparsity = 1 - sum_i |Sel(i)| / (B Hq N (N + 1) / 2), the share
      of causal (query, key) pairs skipped; density = 1 - sparsity;
    * tile density = visited 64 x 64 tiles (diagonal blocks with a visible
      pair plus n_I sparse tiles) over the causal tile count
      B Hq nb (nb + 1) / 2 -- for performance accounting;
    * MSE = mean over all output elements of (o - o_dense)^2 (the pages'
      single-operator MSE against dense attention).
    """
    B, Hq, N = pl.batch, pl.heads_q, pl.seq_len
    S = pl.segment
    nb = N // BLOCK
    total_pairs = B * Hq * N * (N + 1) / 2
    sel = selected_counts(pl, n_I).sum()
    diag_tiles = 0
    for b in range(B):
        for h in range(Hq):
            rows = pl.pi_q[b, h].reshape(nb, BLOCK)
            tI = (np.arange(nb) * BLOCK) // S
            for c in range(S // BLOCK):
                j0 = tI * S + c * BLOCK
                diag_tiles += int((rows.max(axis=1) >= j0).sum())
    out = {
        "pair_sparsity": 1.0 - sel / total_pairs,
        "tile_density": (diag_tiles + int(n_I.sum()))
        / (B * Hq * nb * (nb + 1) / 2),
        "visited_sparse_tiles": int(n_I.sum()),
        "visited_diag_tiles": diag_tiles,
    }
    if o is not None and o_dense is not None:
        out["mse"] = float(np.mean((o - o_dense) ** 2))
    return out
