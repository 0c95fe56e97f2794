// Internal host-side launchers of the gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kHeadDim = 128;        // supported head dimension
constexpr int kBlock = 64;           // query-block rows and key-tile keys
constexpr int kPoolRows = 1024;      // rows per pooling workgroup
constexpr int kScoreRows = 256;      // rows per scoring workgroup (k_key_score
                                     // is written for exactly 256)
constexpr int kSortChunk = 4096;     // elements sorted in LDS by one workgroup
constexpr int kRestrictChunk = 4096; // pi_K entries per restriction workgroup
constexpr int kRestrictSplit = 8;    // restriction workgroups per chunk (t interleaved)
constexpr int kMaxTiles = 2048;      // N / 64 at the largest supported N
// The kernels' thread layouts are written for these values: 16 lanes of 8
// elements per 128-wide row, 64-row blocks matching the 32 x 32 MFMA tiles,
// whole per-thread shares of the restriction and Top-K chunks.
static_assert(kHeadDim == 128 && kBlock == 64, "row and block shapes");
static_assert(kRestrictChunk % 256 == 0, "restriction chunk per 256 threads");
static_assert(kMaxTiles % 64 == 0, "Top-K positions per lane");

struct PlanDims {
  int B, Hq, Hkv, N, S, T, G;
  int n_pool_chunks;      // ceil(N / kPoolRows)
  int n_score_wg;         // ceil(N / kScoreRows)
  int n_restrict_chunks;  // ceil(N / kRestrictChunk)
  size_t list_len;        // S T (T - 1) / 2 entries of L per (b, g)
};

// ---- importance estimator
hipError_t launch_pool_q(const PlanDims& d, const uint16_t* q, int64_t* part,
                         hipStream_t s);
hipError_t launch_pool_reduce(const PlanDims& d, const int64_t* part,
                              int64_t* pooled, hipStream_t s);
hipError_t launch_key_score(const PlanDims& d, const uint16_t* k,
                            const int64_t* pooled, int64_t* vscore,
                            int32_t* blocksum, float* kpart, hipStream_t s);
hipError_t launch_segment_sum(const PlanDims& d, const int32_t* blocksum,
                              int64_t* segsum, const float* kpart,
                              float* kmax2, hipStream_t s);
hipError_t launch_contrast(const PlanDims& d, const uint16_t* k,
                           const int32_t* L, const int64_t* segsum,
                           int64_t* contrast, hipStream_t s);
hipError_t launch_query_score(const PlanDims& d, const uint16_t* q,
                              const int64_t* contrast, int64_t* u,
                              hipStream_t s);

// ---- index builder
// Sorts every segment of `seglen` consecutive scores (n_seg segments) by
// (score descending, index ascending) and writes, for each sorted position,
// the element's index within its row of `rowlen` elements to `out`.
hipError_t launch_segmented_argsort(const int64_t* score, int n_seg,
                                    int seglen, int rowlen, uint64_t* key_a,
                                    int32_t* idx_a, uint64_t* key_b,
                                    int32_t* idx_b, int32_t* out,
                                    hipStream_t s);
hipError_t launch_iota(int32_t* out, size_t n, int rowlen, hipStream_t s);
// Segment-local key order: tile scores of pi_K's 64-key chunks (tscore,
// int64 [B Hkv N / 64]) and the lists L_t (tiles of segments < t by score).
hipError_t launch_segment_tiles(const PlanDims& d, const int64_t* v,
                                const int32_t* pi_k, int64_t* tscore,
                                int32_t* L, hipStream_t s);
hipError_t launch_restrict(const PlanDims& d, const int32_t* pi_k,
                           int32_t* cnt, int32_t* cum, int32_t* L,
                           hipStream_t s);

// ---- stop points (pooled means -> n_I)
// Sum of the 64 query rows of every block of pi_Q: qsum, fp32
// [B, Hq, N / 64, 128].
hipError_t launch_block_qsum(const PlanDims& d, const uint16_t* q,
                             const int32_t* pi_q, float* qsum, hipStream_t s);
struct StopArgs {
  const uint16_t* k;
  const int32_t* L;
  const int32_t* pi_q;
  const float* qsum;
  int32_t* n_I;     // out: [B, Hq, N / 64]
  long long list_len;
  int B, Hq, Hkv, N, S, T, G;
  double tau;
  double c2;        // kappa * log2(e)
  int fixed;        // >= 0: n_I = min(fixed, t S / 64), no scan
};
hipError_t launch_stop_scan(const StopArgs& a, hipStream_t s);

// ---- per-block centroid Top-K selection (instead of the tau stop)
constexpr int kMaskWords = kMaxTiles / 32;  // bitmask words per query block
// the attention kernel reads a block's mask one word per lane
static_assert(kMaskWords == 64, "one Top-K mask word per lane of a wave");
struct TopkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* pi_q;
  const int32_t* L;
  int64_t* scores;   // scratch: per (b, h) and block, one score per tile
  uint32_t* tmask;   // out: [B, Hq, N / 64, kMaskWords] selected positions
  int32_t* n_I;      // out: tiles selected per block
  long long list_len;
  int B, Hq, Hkv, N, S, T, G;
  int K;             // tiles per block (>= 0)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Bytes of the scores scratch: one int64 per (block, tile of its L_t).
size_t topk_scratch_bytes(int B, int Hq, int S, int T);

// Per (b, KV head, segment): its G (S / 64) query blocks by stop point
// descending, for groups of at most kOrderMax blocks.
constexpr int kOrderMax = 1024;
hipError_t launch_block_order(const PlanDims& d, const int32_t* n_I,
                              int32_t* order, hipStream_t s);

// ---- attention
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;      // V as fp16, the copy the PV products read
  const uint16_t* v_in;   // the caller's V (bf16), converted into v
  uint16_t* v16;          // = v, writable (the conversion's output)
  uint16_t* o;
  float* lse;
  const int32_t* pi_q;
  const int32_t* L;
  int32_t* n_I;  // stop points: read; exact mode: tiles attended, written
  long long list_len;
  int B, Hq, Hkv, N, S, T, G;
  int wg_per_group;
  int n_groups;
  float c2;        // kappa * log2(e)
  const float* kmax2;  // per (b, KV head): the largest |k_j|^2 (fp32)
  int32_t* wg_flag;    // per job: 1 = logits unbounded (kMaxRef runs it)
  // Tail pool of the bounded-reference launch (a per-XCD rebalancing of
  // the last groups): slots (per XCD, as in the launch's XCD mapping) from
  // pool_start on are claimed in group order from *pool_ctr, which the
  // local pass clears; pool_extra more workgroups per XCD may claim them.
  // pool_start < 0: no pool.
  int* pool_ctr;
  int pool_start;
  int pool_extra;
  float* lse2;         // per row: the local pass's log2-sum-exp (exp2 domain)
  uint16_t* olo;       // per row: the local output's residual below its bf16
                       // value in O ([B, Hq, N, 128] bf16)
  int local_only;      // 1: the local pass only (no sparse tile visited)
  int local_steps;     // local steps of the sparse passes: always 0
  const int32_t* border;  // per group: blocks by stop point (null: in order)
  int exact;       // 1: exact per-block max test instead of the stop points
  float exact_thr; // that test's threshold on the raw dot products (theta / kappa)
  int topk;        // 1: per-block Top-K masks instead of the stop points
  const uint32_t* tmask;  // [B, Hq, N / 64, kMaskWords]: Top-K selections
};
// The local pass (V converted to fp16, then every row's dense local window,
// rows in their own order; needs nothing from the plan but its workspace)
// and the sparse passes (after the local pass and the stop points).
hipError_t launch_attention_local(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_sparse(const AttnArgs& a, hipStream_t s);
// Query blocks one attention workgroup processes (sets wg_per_group).
int attention_blocks_per_wg();
// The tail pool's settings for the launch shape in `a`.
void set_tail_pool(AttnArgs& a);

}  // namespace sa
