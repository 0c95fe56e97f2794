/*
 * sparse_attn.h -- C ABI of the permuted, early-stopping block-sparse causal
 * prefill attention library (libsparse_attn.so, gfx950 / MI355X).
 *
 * The method is the one described on the page "S2O: Early Stopping for
 * Sparse Attention via Online Permutation" (Summary): lightweight index
 * arrays -- a segment-local query ordering and a global key/value ordering
 * ranked by stripe-level mean pooling -- are built without moving any
 * tensor; the kernel gathers the indexed tokens into on-chip memory, visits
 * key/value blocks from most to least important and stops once a block's
 * score falls under a threshold tau. Dense attention is Eq. (1) of the page
 * "AB-Sparse: Sparse Attention with Adaptive Block Size ..." (softmax of
 * q.k/sqrt(d) over the causal prefix).
 *
 * Two calls make up the path:
 *   sparse_attn_plan     -- the importance estimator and the index builder
 *                           (both orders and the causally restricted key
 *                           lists, integer-exact) and the stop points of
 *                           the tau stop, scanned from pooled means;
 *   sparse_attn_prefill  -- the gather attention kernel, which stops each
 *                           query block at its stop point, and the scatter
 *                           of each output row back to its original
 *                           position.
 * sparse_attn_forward makes both in one call, overlapping the prefill's
 * dense local windows (which need only q, k, v) with the plan on a second
 * stream.
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned DEVICE pointers, bfloat16 (raw 16-bit
 *     patterns), contiguous: Q and O are [batch, heads_q, seq_len, head_dim],
 *     K and V are [batch, heads_kv, seq_len, head_dim]. Query head h reads
 *     KV head h / (heads_q / heads_kv).
 *   - Work is enqueued on the caller's stream and runs asynchronously; no
 *     entry point synchronizes except sparse_attn_plan_export.
 *   - Every argument is validated before anything is launched; a call that
 *     returns a validation error has launched nothing and changed nothing.
 *   - Status codes, never exceptions or aborts. A HIP launch failure is
 *     reported as SA_ERR_HIP (work launched before it stays enqueued);
 *     errors of earlier asynchronous work may surface there too. Non-finite
 *     inputs give unspecified (but memory-safe) results.
 *   - No global state: all device scratch lives in the caller's workspace.
 *     A plan must not be used on two streams at once (sparse_attn_forward
 *     orders its own two streams).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SA_OK                        0
#define SA_ERR_INVALID_ARG          (-1)  /* bad value (tau < 0 or NaN, ...) */
#define SA_ERR_UNSUPPORTED_SHAPE    (-2)  /* shape outside the limits below  */
#define SA_ERR_WORKSPACE_TOO_SMALL  (-3)
#define SA_ERR_HIP                  (-4)  /* a HIP runtime call failed       */
#define SA_ERR_NULL_POINTER         (-5)
#define SA_ERR_HOST_ALLOC           (-6)  /* the small host plan object     */

/* Flags (sa_params.flags). */
#define SA_NO_QPERM      1u   /* identity query order (ablation)             */
#define SA_NO_KVPERM     2u   /* identity key/value order (ablation)         */
#define SA_NO_EARLYSTOP  4u   /* visit every tile (same result as tau = 0)   */
/* Dense local window only: every query block attends to its own segment
 * (causal) and to no tile of L_t; n_I = 0 everywhere. The baseline of the
 * S2O page's component ablation (Key points: keeping only the dense local
 * window). Takes precedence over SA_NO_EARLYSTOP. */
#define SA_LOCAL_ONLY    8u
/* Segment-local key/value order (the PBS-Attn page's permutation inside
 * causal segments, abstract): pi_K sorts the keys of each segment by their
 * stripe score (descending, ties by index); its 64-key chunks are the tiles,
 * and segment t visits the tiles of segments 0 .. t - 1 by tile score (sum
 * of the scores of its keys) descending, ties by tile index. L_t keeps its
 * layout. SA_NO_KVPERM takes precedence; sparse_attn_plan_set_kv_order
 * returns SA_ERR_INVALID_ARG for a plan built with this flag. */
#define SA_SEGMENT_KV   16u

/*
 * Problem description.
 *   block    must be 64 (query-block and key-tile size);
 *   head_dim must be 128;
 *   segment  S: a multiple of 64 that divides seq_len;
 *   seq_len  N: at most 131072 (2^17) -- the bound under which the int64
 *            ranking scores cannot overflow;
 *   heads_q  a multiple of heads_kv, heads_q / heads_kv <= 256;
 *   tau      the stop threshold, a finite value >= 0 (tau = 0 never stops;
 *            tau >= 1 stops before the first sparse tile).
 * All sizes must be positive.
 */
typedef struct sa_params {
    int32_t  batch;
    int32_t  heads_q;
    int32_t  heads_kv;
    int32_t  seq_len;
    int32_t  head_dim;
    int32_t  segment;
    int32_t  block;
    double   tau;
    uint32_t flags;
} sa_params;

/* Opaque host-side plan object. It refers into the caller's workspace (it
 * does not own device memory) and must not outlive it. */
typedef struct sa_plan sa_plan;

/*
 * Bytes of device workspace a plan for *p needs (0 if *p is invalid). The
 * workspace holds the index arrays (global KV order, restricted key lists,
 * query order, stop points) and the planner's scratch (pooled sums, scores,
 * sort buffers). Its size depends only on the shape, never on the data.
 */
size_t sparse_attn_workspace_bytes(const sa_params* p);

/*
 * The importance estimator and the index builder (S2O page, Summary: the
 * segment-local query ordering and the global key/value ordering ranked by
 * stripe-level mean pooling). Enqueues, on `stream`:
 *   1. pooled group query P = sum of the fixed-point images fx(q) =
 *      clamp(rint(256 q), -32768, 32767) over all queries of each KV group;
 *   2. key stripe scores v_j = P . fx(k_j) (int64);
 *   3. global KV order pi_K: v descending, ties by index;
 *   4. restricted lists L_t = pi_K without keys >= t*S, for t = 1..T-1;
 *   5. contrast vectors C_t = t S * sum_{j in L_t[0:64]} fx(k_j)
 *                            - 64 * sum_{j < t S} fx(k_j);
 *   6. query scores u_i = fx(q_i) . C_seg(i) (0 in segment 0);
 *   7. segment-local query order pi_Q: u descending, ties by index;
 *   8. the stop point n_I of every query block for the plan's tau (the rule
 *      is stated at sparse_attn_prefill): every estimate there is a mean
 *      logit, equal to (sum of the block's 64 queries) . (sum of the 64
 *      keys) / 4096, so n_I follows from fp32 sums of the blocks' queries
 *      and of the keys of the local blocks and of the tiles of L_t, with
 *      the running total and the test in float64.
 * All scores of steps 1-7 are exact integers, so the orders are
 * reproducible bit for bit.
 * q, k: device pointers (see conventions); workspace: device buffer of at
 * least sparse_attn_workspace_bytes(p) bytes, 256-byte aligned. On success
 * *out receives a new plan (free with sparse_attn_plan_destroy).
 */
int sparse_attn_plan(const sa_params* p, const void* q, const void* k,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream, sa_plan** out);

/*
 * The attention (S2O page, Summary: fetch the indexed tokens into on-chip
 * memory, process blocks from most to least important, stop once a block's
 * score falls under tau). For each 64-row query block I (rows
 * pi_Q[64 I .. 64 I + 63], all in segment t):
 *   - the dense local window: exact causal attention against the keys of
 *     segment t, and its estimated mass
 *     E_diag = sum_c (n_vis(I, c) / 64) exp(kappa * mean logit of block c);
 *   - the sparse tiles T_k = L_t[64 k .. 64 k + 63], k = 0, 1, ...: estimate
 *     E_k = 64 exp(kappa * mean logit of the 64 x 64 tile), stop at the
 *     first k with E_k / (E_diag + E_0 + ... + E_k) < tau, otherwise attend
 *     to the tile (online softmax);
 *   - each output row is written to its original position in O.
 * kappa = 1/sqrt(head_dim). q, k must be the tensors the plan was built
 * from (not checked: the stop points, and the plan's bound on the key norms
 * that keeps the softmax's exponentials finite, come from them). v: the
 * value products run in fp16 (weights rounded to fp16, V converted into
 * the workspace, exactly for entries of magnitude in [2^-14, 65504]);
 * entries beyond 65504 in magnitude give unspecified results. o: device
 * [batch, heads_q, seq_len, 128] bfloat16, fully overwritten (each value
 * rounded to bfloat16 once, from fp32). lse (may be NULL): device
 * [batch, heads_q, seq_len] float32, natural-log log-sum-exp of kappa q.k
 * over each row's key set.
 * The stop points come from the plan (export N_I). After a setter below or
 * sparse_attn_plan_set_kv_order changed what they depend on, this call
 * first rescans them on `stream` (one extra launch), then launches the
 * attention: two launches of one kernel, the second running only the
 * workgroups whose logits are too large to be provably bounded. A plan must
 * not be used by two calls at once.
 */
int sparse_attn_prefill(const sa_plan* plan, const void* q, const void* k,
                        const void* v, void* o, float* lse,
                        hipStream_t stream);

/*
 * sparse_attn_plan followed by sparse_attn_prefill in one call, with the
 * same results: the prefill's dense local windows depend on q, k, v alone,
 * so they run on side_stream (after the work already enqueued on `stream`)
 * while the planner runs on `stream`; the rest of the attention waits on
 * `stream` for both. Arguments as for the two calls; side_stream must
 * belong to the same device and may equal `stream` (then everything runs
 * in order on `stream`). On return the work is enqueued on both streams
 * and `stream` is ordered after all of it; o, lse and the workspace must
 * stay allocated until it completes. On success *out receives the plan
 * (setters, exports and further prefills as from sparse_attn_plan; free
 * with sparse_attn_plan_destroy).
 */
int sparse_attn_forward(const sa_params* p, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream,
                        hipStream_t side_stream, sa_plan** out);

/* For callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid it): the same
 * results as sparse_attn_forward with side_stream == stream (plan, then
 * prefill, all on `stream`, which must belong to the current device), with
 * the workspace taken from a fixed device array of SA_STATIC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.
 * No plan object is returned and nothing is allocated (no device memory, no
 * host memory, no events). Arguments as for sparse_attn_forward; a shape
 * whose workspace (sparse_attn_workspace_bytes) exceeds
 * SA_STATIC_SCRATCH_BYTES returns SA_ERR_WORKSPACE_TOO_SMALL before
 * anything is launched. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and give
 * unspecified results; calls in stream order do not interfere. */
#define SA_STATIC_SCRATCH_BYTES (256ull << 20)
int sparse_attn_forward_static(const sa_params* p, const void* q,
                               const void* k, const void* v, void* o,
                               float* lse, hipStream_t stream);

/* Change the threshold of an existing plan (the index arrays do not depend
 * on tau). Returns SA_ERR_INVALID_ARG for tau < 0 or NaN. */
int sparse_attn_plan_set_tau(sa_plan* plan, double tau);

/* Fixed tile budget instead of the tau stop: with tiles >= 0 every query
 * block of segment t visits the first min(tiles, t S / 64) tiles of L_t
 * (the most important tiles of the mean-pooled ranking, the same count for
 * every block -- the fixed-budget selection the S2O page compares its
 * adaptive stop with, Key points); tiles < 0 restores the tau stop (the
 * default). n_I records the count. SA_LOCAL_ONLY still visits no tile. */
int sparse_attn_plan_set_budget(sa_plan* plan, int32_t tiles);

/* Exact per-block maximum test instead of the tau stop (the BSFA page,
 * abstract: exact query-key scores, a block is skipped when its maximum
 * score is under a threshold; the page calibrates one per layer and head,
 * here it is given). With theta not NaN every tile of L_t is scored
 * exactly and attended iff max over its 64 x 64 logits kappa q . k >= theta
 * (+inf: none, -inf: all); the dense local window is always attended and
 * n_I counts the attended tiles. theta = NaN (the default) restores the tau
 * stop. Takes precedence over a budget; SA_LOCAL_ONLY still visits no
 * tile. */
int sparse_attn_plan_set_max_threshold(sa_plan* plan, double theta);

/* Per-block Top-K tile selection from mean-pooled centroids instead of the
 * tau stop (the AB-Sparse page's block-sparse workflow, the paragraph
 * around its Figure 2 and the footnote on mean pooling: key blocks scored
 * by the product of the query with their centroid, the best K attended).
 * With tiles >= 0, every query block I of segment t >= 1 scores each tile
 * T_k of L_t by r = (sum of fx(q) over I's 64 rows) . (sum of fx(k) over
 * T_k's 64 keys) -- exact integers, fx as in sparse_attn_plan -- and
 * attends to the min(tiles, t S / 64) tiles of highest r, ties by smaller
 * position in L_t; the dense local window is always attended and n_I
 * counts the selected tiles. The scoring (an fp64 MFMA contraction per
 * segment, exact) and the selection are enqueued on `stream` by this call;
 * `scratch` (device, 8-byte aligned, at least
 * sparse_attn_topk_scratch_bytes(plan) bytes: one int64 per block and
 * tile) is used only by that work. The selections stay with the plan until
 * the next call of this function or of sparse_attn_plan_set_kv_order
 * (which ends the mode). tiles < 0 restores the tau stop (scratch may then
 * be NULL). The exact maximum test takes precedence; SA_LOCAL_ONLY still
 * visits no tile. Returns SA_ERR_WORKSPACE_TOO_SMALL for a short scratch. */
size_t sparse_attn_topk_scratch_bytes(const sa_plan* plan);
int sparse_attn_plan_set_topk(sa_plan* plan, int32_t tiles, void* scratch,
                              size_t scratch_bytes, hipStream_t stream);

/* What sparse_attn_plan_export copies (element type, count). */
#define SA_EXPORT_PI_K         0  /* int32 [B, Hkv, N]                        */
#define SA_EXPORT_PI_Q         1  /* int32 [B, Hq, N]                         */
#define SA_EXPORT_L            2  /* int32 [B, Hkv, S T (T-1) / 2]: L_1, L_2,..*/
#define SA_EXPORT_N_I          3  /* int32 [B, Hq, N / 64]: stop points       */
#define SA_EXPORT_KEY_SCORE    4  /* int64 [B, Hkv, N]: v                     */
#define SA_EXPORT_QUERY_SCORE  5  /* int64 [B, Hq, N]: u                      */
#define SA_EXPORT_CONTRAST     6  /* int64 [B, Hkv, T, 128]: C (t = 0 zero)   */
#define SA_EXPORT_POOLED       7  /* int64 [B, Hkv, 128]: P                   */
#define SA_EXPORT_TOPK_MASK    8  /* uint32 [B, Hq, N / 64, 64]: Top-K tiles  */
                                  /* selected (bit p of word w: position    */
                                  /* 32 w + p of L_t)                        */

/* Bytes of one export (0 for an unknown `what`). */
size_t sparse_attn_plan_export_bytes(const sa_plan* plan, int what);

/* Copy one plan array to host memory `host_dst` (at least
 * sparse_attn_plan_export_bytes bytes) after the work enqueued on `stream`
 * so far; synchronizes `stream`. N_I holds the stop points after
 * sparse_attn_plan (and after every prefill), and after a prefill with the
 * exact maximum test the number of tiles each block attended. */
int sparse_attn_plan_export(const sa_plan* plan, int what, void* host_dst,
                            size_t bytes, hipStream_t stream);

/* Replace the global KV order by `pi_k` (device int32 [B, Hkv, N], each row
 * a permutation of 0..N-1, not checked) and rebuild everything that depends
 * on it (restricted lists, contrast vectors, query scores and order). For
 * tests: with tau = 0 the output must not depend on the KV order.
 * Returns SA_ERR_INVALID_ARG for a plan built with SA_SEGMENT_KV. */
int sparse_attn_plan_set_kv_order(sa_plan* plan, const void* pi_k,
                                  hipStream_t stream);

/* Free the host plan object (the workspace stays the caller's). NULL-safe. */
void sparse_attn_plan_destroy(sa_plan* plan);

/* Static string describing a status code. */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
