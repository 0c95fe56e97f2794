"""CPU oracle for permuted, early-stopping block-sparse causal prefill attention.

TEST INFRASTRUCTURE. This package is the slow, plain reference that the GPU
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product package
(``permuted_block_sparse_amd``) never imports it, and it imports nothing from
the product: the two share no kernels, helpers, constants or tables. Its only
inputs are bfloat16 bit patterns (``uint16`` arrays) produced by the seeded
generator in ``synthetic/``.

Arithmetic: int64 for every ranking score (exact), float64 for everything
real, computed from the exact values of the bfloat16 inputs.

Pinned parts (see tests/test_oracle_*.py):
  * dense causal attention (Eq. (1) of the AB-Sparse page) -- against torch's
    float64 scaled-dot-product attention, closed forms and causality;
  * the S2O steps -- tau = 0 reproduces dense attention for every flag
    combination and for any key/value order; one segment reproduces dense
    attention for any tau; a closed form for the stop point with constant
    keys; brute-force restricted attention on tiny inputs; brute-force
    ranking of the two orders; worked examples of both orders; a golden
    fixture in tests/golden/;
  * the dense-local-window-only baseline (SA_LOCAL_ONLY) -- against dense
    attention of each segment taken as a sequence of its own;
  * attention recall -- equal to 1 when nothing is skipped, to the
    logsumexp difference of the selected and the full causal key sets
    (library logsumexp), and to the own-segment share for SA_LOCAL_ONLY;
  * the segment-local key order (SA_SEGMENT_KV) -- a hand-derived example
    of the tile order, invariants, and tau = 0 reproducing dense attention;
  * the exact per-block maximum test -- tile maxima by brute force (library
    einsum), theta = -inf / +inf reproducing dense / local-only attention,
    monotone selection in theta;
  * the per-block centroid Top-K selection -- tile scores as sums of the
    integer logit matrix with ranks counted pairwise, a hand-derived case in
    which blocks of one segment choose different tiles (and ties), K = 0 /
    K >= all reproducing local-only / dense attention;
  * the metrics -- selected-set sizes against explicit per-row key sets,
    closed forms of pair sparsity and tile density, MSE against torch.
Parity unpinned: the agreement of the sparsity/MSE figures with the numbers
printed on the S2O summary page (those need real models and datasets).
"""
from .s2o import (SA_NO_QPERM, SA_NO_KVPERM, SA_NO_EARLYSTOP, SA_LOCAL_ONLY,
                  SA_SEGMENT_KV,
                  Plan, decode_bf16, fixed_point, dense_causal, plan,
                  stop_points, attend, recall, exact_max_selection,
                  topk_selection, s2o_attention,
                  selected_counts, metrics, restricted_list, kappa_of)

__all__ = ["SA_NO_QPERM", "SA_NO_KVPERM", "SA_NO_EARLYSTOP", "SA_LOCAL_ONLY",
           "SA_SEGMENT_KV",
           "Plan", "decode_bf16", "fixed_point", "dense_causal", "plan",
           "stop_points", "attend", "recall", "exact_max_selection",
           "topk_selection", "s2o_attention",
           "selected_counts", "metrics", "restricted_list", "kappa_of"]
