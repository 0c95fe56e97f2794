// Host side of libsparse_attn: argument validation, workspace layout and the
// launch sequence behind the C ABI declared in include/sparse_attn.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>

#include "sa_launch.h"
#include "sparse_attn.h"

using namespace sa;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Offsets of every array inside the caller's workspace.
struct Layout {
  size_t pool_part, pooled, vscore, blocksum, segsum, contrast, u;
  size_t key_a, idx_a, key_b, idx_b;
  size_t pi_k, L, pi_q, n_I, rcnt, rcum, qsum, kpart, kmax2, wg_flag, lse2,
      border, olo, v16, tmask, pool;
  size_t total;
};

int validate(const sa_params* p) {
  if (p == nullptr) return SA_ERR_NULL_POINTER;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 ||
      p->seq_len <= 0 || p->head_dim <= 0 || p->segment <= 0 || p->block <= 0)
    return SA_ERR_UNSUPPORTED_SHAPE;
  if (p->block != kBlock || p->head_dim != kHeadDim)
    return SA_ERR_UNSUPPORTED_SHAPE;
  if (p->segment % kBlock != 0 || p->seq_len % p->segment != 0)
    return SA_ERR_UNSUPPORTED_SHAPE;
  if (p->seq_len > (1 << 17)) return SA_ERR_UNSUPPORTED_SHAPE;
  if (p->heads_q % p->heads_kv != 0 || p->heads_q / p->heads_kv > 256)
    return SA_ERR_UNSUPPORTED_SHAPE;
  // every (b, h) row of Q and every sorted segment must index with int32
  if ((long long)p->batch * p->heads_q * p->seq_len > (1ll << 31) / 2)
    return SA_ERR_UNSUPPORTED_SHAPE;
  if (!(p->tau >= 0.0) || std::isinf(p->tau)) return SA_ERR_INVALID_ARG;
  if (p->flags &
      ~(SA_NO_QPERM | SA_NO_KVPERM | SA_NO_EARLYSTOP | SA_LOCAL_ONLY |
        SA_SEGMENT_KV))
    return SA_ERR_INVALID_ARG;
  return SA_OK;
}

PlanDims dims_of(const sa_params* p) {
  PlanDims d;
  d.B = p->batch;
  d.Hq = p->heads_q;
  d.Hkv = p->heads_kv;
  d.N = p->seq_len;
  d.S = p->segment;
  d.T = p->seq_len / p->segment;
  d.G = p->heads_q / p->heads_kv;
  d.n_pool_chunks = (d.N + kPoolRows - 1) / kPoolRows;
  d.n_score_wg = (d.N + kScoreRows - 1) / kScoreRows;
  d.n_restrict_chunks = (d.N + kRestrictChunk - 1) / kRestrictChunk;
  d.list_len = (size_t)d.S * d.T * (d.T - 1) / 2;
  return d;
}

// Workgroups of one attention launch: per (b, KV head, segment), the G
// heads' query blocks of the segment, attention_blocks_per_wg() at a time.
size_t attention_workgroups(const PlanDims& d) {
  const int qblocks = d.G * (d.S / kBlock);
  const int bpw = attention_blocks_per_wg();
  return (size_t)d.B * d.Hkv * d.T * ((qblocks + bpw - 1) / bpw);
}

Layout layout_of(const PlanDims& d) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t nbg = (size_t)d.B * d.Hkv, nbh = (size_t)d.B * d.Hq;
  const size_t nsort = nbh * d.N;  // >= nbg * N
  L.pool_part = take(nbh * d.n_pool_chunks * kHeadDim * sizeof(int64_t));
  L.pooled = take(nbg * kHeadDim * sizeof(int64_t));
  L.vscore = take(nbg * d.N * sizeof(int64_t));
  L.blocksum = take(nbg * (d.N / kBlock) * kHeadDim * sizeof(int32_t));
  L.segsum = take(nbg * d.T * kHeadDim * sizeof(int64_t));
  L.contrast = take(nbg * d.T * kHeadDim * sizeof(int64_t));
  L.u = take(nbh * d.N * sizeof(int64_t));
  L.key_a = take(nsort * sizeof(uint64_t));
  L.idx_a = take(nsort * sizeof(int32_t));
  L.key_b = take(nsort * sizeof(uint64_t));
  L.idx_b = take(nsort * sizeof(int32_t));
  L.pi_k = take(nbg * d.N * sizeof(int32_t));
  L.L = take(nbg * (d.list_len > 0 ? d.list_len : 1) * sizeof(int32_t));
  L.pi_q = take(nbh * d.N * sizeof(int32_t));
  L.n_I = take(nbh * (d.N / kBlock) * sizeof(int32_t));
  L.rcnt = take(nbg * d.n_restrict_chunks * d.T * sizeof(int32_t));
  L.rcum = take(nbg * d.n_restrict_chunks * d.T * sizeof(int32_t));
  L.qsum = take(nbh * (d.N / kBlock) * kHeadDim * sizeof(float));
  L.kpart = take(nbg * d.n_score_wg * sizeof(float));
  L.kmax2 = take(nbg * sizeof(float));
  L.wg_flag = take(attention_workgroups(d) * sizeof(int32_t));
  L.lse2 = take(nbh * d.N * sizeof(float));
  L.border = take(nbh * (d.N / kBlock) * sizeof(int32_t));
  L.olo = take(nbh * d.N * kHeadDim * sizeof(uint16_t));
  L.v16 = take(nbg * d.N * kHeadDim * sizeof(uint16_t));
  L.tmask = take(nbh * (d.N / kBlock) * kMaskWords * sizeof(uint32_t));
  L.pool = take(sizeof(int32_t));
  L.total = off;
  return L;
}

}  // namespace

struct sa_plan {
  sa_params p;
  int32_t budget = -1;  // >= 0: fixed tile budget instead of the tau stop
  int32_t topk = -1;    // >= 0: per-block Top-K selections (masks selected)
  double max_theta = std::numeric_limits<double>::quiet_NaN();  // exact test
  // n_I holds the stop points of the current settings (set by the stop
  // scan; cleared by every setter and by an exact-mode prefill, whose n_I
  // counts attended tiles)
  mutable bool stops_valid = false;
  PlanDims d;
  Layout lay;
  char* ws;
  const void* q;
  const void* k;

  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
};

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

// Everything that depends on the global KV order: restricted lists,
// contrast vectors, query scores and the query order.
bool segment_kv(const sa_params& p) {
  return (p.flags & SA_SEGMENT_KV) && !(p.flags & SA_NO_KVPERM);
}

int build_from_kv_order(sa_plan* pl, hipStream_t s) {
  const PlanDims& d = pl->d;
  hipError_t e;
  if (segment_kv(pl->p)) {
    // tile scores go to the first sort buffer, free until the query sort
    e = launch_segment_tiles(d, pl->at<int64_t>(pl->lay.vscore),
                             pl->at<int32_t>(pl->lay.pi_k),
                             pl->at<int64_t>(pl->lay.key_a),
                             pl->at<int32_t>(pl->lay.L), s);
  } else {
    e = launch_restrict(d, pl->at<int32_t>(pl->lay.pi_k),
                        pl->at<int32_t>(pl->lay.rcnt),
                        pl->at<int32_t>(pl->lay.rcum),
                        pl->at<int32_t>(pl->lay.L), s);
  }
  if (e != hipSuccess) return SA_ERR_HIP;
  e = launch_contrast(d, static_cast<const uint16_t*>(pl->k),
                      pl->at<int32_t>(pl->lay.L),
                      pl->at<int64_t>(pl->lay.segsum),
                      pl->at<int64_t>(pl->lay.contrast), s);
  if (e != hipSuccess) return SA_ERR_HIP;
  e = launch_query_score(d, static_cast<const uint16_t*>(pl->q),
                         pl->at<int64_t>(pl->lay.contrast),
                         pl->at<int64_t>(pl->lay.u), s);
  if (e != hipSuccess) return SA_ERR_HIP;
  const size_t nbh = (size_t)d.B * d.Hq;
  if (pl->p.flags & SA_NO_QPERM) {
    e = launch_iota(pl->at<int32_t>(pl->lay.pi_q), nbh * d.N, d.N, s);
  } else {
    e = launch_segmented_argsort(
        pl->at<int64_t>(pl->lay.u), (int)(nbh * d.T), d.S, d.N,
        pl->at<uint64_t>(pl->lay.key_a), pl->at<int32_t>(pl->lay.idx_a),
        pl->at<uint64_t>(pl->lay.key_b), pl->at<int32_t>(pl->lay.idx_b),
        pl->at<int32_t>(pl->lay.pi_q), s);
  }
  if (e != hipSuccess) return SA_ERR_HIP;
  // the blocks' query sums, for the stop scan
  e = launch_block_qsum(d, static_cast<const uint16_t*>(pl->q),
                        pl->at<int32_t>(pl->lay.pi_q),
                        pl->at<float>(pl->lay.qsum), s);
  return hip_status(e);
}

bool exact_mode(const sa_plan* pl) {
  return !std::isnan(pl->max_theta) && !(pl->p.flags & SA_LOCAL_ONLY);
}

bool topk_mode(const sa_plan* pl) {
  return pl->topk >= 0 && !exact_mode(pl) && !(pl->p.flags & SA_LOCAL_ONLY);
}

// The sparse pass takes each group's blocks by stop point (small groups).
bool block_order_used(const PlanDims& d) {
  return d.G * (d.S / kBlock) <= kOrderMax;
}

// n_I of the plan's current settings: the tau stop scanned from pooled
// means, or a fixed count (dense local window only: 0; fixed budget K:
// min(K, t S / 64); tau = 0 or SA_NO_EARLYSTOP: every tile of L_t).
int run_stop_scan(const sa_plan* pl, hipStream_t s) {
  const PlanDims& d = pl->d;
  StopArgs a;
  a.k = static_cast<const uint16_t*>(pl->k);
  a.L = pl->at<int32_t>(pl->lay.L);
  a.pi_q = pl->at<int32_t>(pl->lay.pi_q);
  a.qsum = pl->at<float>(pl->lay.qsum);
  a.n_I = pl->at<int32_t>(pl->lay.n_I);
  a.list_len = (long long)d.list_len;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.S = d.S;
  a.T = d.T;
  a.G = d.G;
  a.tau = pl->p.tau;
  a.c2 = 1.4426950408889634074 / std::sqrt((double)kHeadDim);
  if (pl->p.flags & SA_LOCAL_ONLY)
    a.fixed = 0;
  else if (pl->budget >= 0)
    a.fixed = pl->budget;
  else if ((pl->p.flags & SA_NO_EARLYSTOP) || pl->p.tau == 0.0)
    a.fixed = std::numeric_limits<int>::max();
  else
    a.fixed = -1;
  hipError_t e = launch_stop_scan(a, s);
  if (e == hipSuccess && block_order_used(d))
    e = launch_block_order(d, a.n_I, pl->at<int32_t>(pl->lay.border), s);
  if (e != hipSuccess) return SA_ERR_HIP;
  pl->stops_valid = true;
  return SA_OK;
}

}  // namespace

// Scratch of sparse_attn_forward_static, for callers that cannot
// allocate: one fixed array per GPU, held until the process ends. In host
// code the array's name is only a stand-in; its device address on the
// current GPU comes from hipGetSymbolAddress (kept per device, taken on the
// first call on that device) and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// The scratch array's device address on the current device.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess ||
        addr == nullptr)
      return SA_ERR_HIP;
    g_scratch_addr[dev] = addr;
  }
  *out = g_scratch_addr[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

size_t sparse_attn_workspace_bytes(const sa_params* p) {
  if (validate(p) != SA_OK) return 0;
  return layout_of(dims_of(p)).total;
}

namespace {

// A plan object over a workspace (validated by the caller).
void plan_fill(sa_plan* pl, const sa_params* p, const void* q, const void* k,
               void* workspace) {
  pl->p = *p;
  pl->d = dims_of(p);
  pl->lay = layout_of(pl->d);
  pl->ws = static_cast<char*>(workspace);
  pl->q = q;
  pl->k = k;
}

// Validation and the plan object (host only; no launch).
int plan_create(const sa_params* p, const void* q, const void* k,
                void* workspace, size_t workspace_bytes, sa_plan** out) {
  if (out == nullptr) return SA_ERR_NULL_POINTER;
  *out = nullptr;
  const int st = validate(p);
  if (st != SA_OK) return st;
  if (q == nullptr || k == nullptr || workspace == nullptr)
    return SA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return SA_ERR_INVALID_ARG;
  const PlanDims d = dims_of(p);
  const Layout lay = layout_of(d);
  if (workspace_bytes < lay.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  sa_plan* pl = new (std::nothrow) sa_plan;
  if (pl == nullptr) return SA_ERR_HOST_ALLOC;
  plan_fill(pl, p, q, k, workspace);
  *out = pl;
  return SA_OK;
}

// Every planner kernel of a new plan: pooling, scores, both orders, the
// restricted lists, the contrast vectors, the stop points.
int plan_launch(sa_plan* pl, hipStream_t stream) {
  const PlanDims& d = pl->d;
  const Layout& lay = pl->lay;
  const sa_params* p = &pl->p;
  const uint16_t* qb = static_cast<const uint16_t*>(pl->q);
  const uint16_t* kb = static_cast<const uint16_t*>(pl->k);
  hipError_t e = launch_pool_q(d, qb, pl->at<int64_t>(lay.pool_part), stream);
  if (e == hipSuccess)
    e = launch_pool_reduce(d, pl->at<int64_t>(lay.pool_part),
                           pl->at<int64_t>(lay.pooled), stream);
  if (e == hipSuccess)
    e = launch_key_score(d, kb, pl->at<int64_t>(lay.pooled),
                         pl->at<int64_t>(lay.vscore),
                         pl->at<int32_t>(lay.blocksum),
                         pl->at<float>(lay.kpart), stream);
  if (e == hipSuccess)
    e = launch_segment_sum(d, pl->at<int32_t>(lay.blocksum),
                           pl->at<int64_t>(lay.segsum),
                           pl->at<float>(lay.kpart), pl->at<float>(lay.kmax2),
                           stream);
  if (e == hipSuccess) {
    const size_t nbg = (size_t)d.B * d.Hkv;
    if (p->flags & SA_NO_KVPERM)
      e = launch_iota(pl->at<int32_t>(lay.pi_k), nbg * d.N, d.N, stream);
    else if (segment_kv(*p))
      e = launch_segmented_argsort(
          pl->at<int64_t>(lay.vscore), (int)(nbg * d.T), d.S, d.N,
          pl->at<uint64_t>(lay.key_a), pl->at<int32_t>(lay.idx_a),
          pl->at<uint64_t>(lay.key_b), pl->at<int32_t>(lay.idx_b),
          pl->at<int32_t>(lay.pi_k), stream);
    else
      e = launch_segmented_argsort(
          pl->at<int64_t>(lay.vscore), (int)nbg, d.N, d.N,
          pl->at<uint64_t>(lay.key_a), pl->at<int32_t>(lay.idx_a),
          pl->at<uint64_t>(lay.key_b), pl->at<int32_t>(lay.idx_b),
          pl->at<int32_t>(lay.pi_k), stream);
  }
  int rc = hip_status(e);
  if (rc == SA_OK) rc = build_from_kv_order(pl, stream);
  if (rc == SA_OK) rc = run_stop_scan(pl, stream);
  return rc;
}

// The attention launches' arguments for the plan's current settings.
AttnArgs attn_args(const sa_plan* plan, const void* q, const void* k,
                   const void* v, void* o, float* lse) {
  const PlanDims& d = plan->d;
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.v16 = plan->at<uint16_t>(plan->lay.v16);
  a.v = a.v16;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.pi_q = plan->at<int32_t>(plan->lay.pi_q);
  a.L = plan->at<int32_t>(plan->lay.L);
  a.n_I = plan->at<int32_t>(plan->lay.n_I);
  a.list_len = (long long)d.list_len;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.S = d.S;
  a.T = d.T;
  a.G = d.G;
  const int qblocks = d.G * (d.S / kBlock);
  const int bpw = attention_blocks_per_wg();
  a.wg_per_group = (qblocks + bpw - 1) / bpw;
  a.n_groups = d.B * d.Hkv * d.T;
  // the exact max test takes precedence over a budget and over tau; the
  // dense local window only takes precedence over everything
  a.exact = exact_mode(plan) ? 1 : 0;
  a.exact_thr = a.exact ? (float)(plan->max_theta *
                                  std::sqrt((double)kHeadDim))
                        : 0.f;
  a.c2 = (float)(1.4426950408889634074 / std::sqrt((double)kHeadDim));
  a.kmax2 = plan->at<float>(plan->lay.kmax2);
  a.wg_flag = plan->at<int32_t>(plan->lay.wg_flag);
  a.lse2 = plan->at<float>(plan->lay.lse2);
  a.olo = plan->at<uint16_t>(plan->lay.olo);
  a.local_only = (plan->p.flags & SA_LOCAL_ONLY) ? 1 : 0;
  a.local_steps = 0;
  a.topk = topk_mode(plan) ? 1 : 0;
  a.tmask = plan->at<uint32_t>(plan->lay.tmask);
  a.border = (!a.exact && !a.topk && block_order_used(d))
                 ? plan->at<int32_t>(plan->lay.border)
                 : nullptr;
  a.pool_ctr = plan->at<int>(plan->lay.pool);
  set_tail_pool(a);
  return a;
}

// The sparse passes, after rescanning stale stop points.
int sparse_passes(const sa_plan* plan, const AttnArgs& a, hipStream_t stream) {
  if (!a.exact && !a.topk && !plan->stops_valid) {
    const int rc = run_stop_scan(plan, stream);
    if (rc != SA_OK) return rc;
  }
  if (a.exact) plan->stops_valid = false;
  return hip_status(launch_attention_sparse(a, stream));
}

}  // namespace

int sparse_attn_plan(const sa_params* p, const void* q, const void* k,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream, sa_plan** out) {
  if (out == nullptr) return SA_ERR_NULL_POINTER;
  *out = nullptr;
  sa_plan* pl = nullptr;
  int rc = plan_create(p, q, k, workspace, workspace_bytes, &pl);
  if (rc != SA_OK) return rc;
  rc = plan_launch(pl, stream);
  if (rc != SA_OK) {
    delete pl;
    return rc;
  }
  *out = pl;
  return SA_OK;
}

int sparse_attn_prefill(const sa_plan* plan, const void* q, const void* k,
                        const void* v, void* o, float* lse,
                        hipStream_t stream) {
  if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr ||
      o == nullptr)
    return SA_ERR_NULL_POINTER;
  const AttnArgs a = attn_args(plan, q, k, v, o, lse);
  const int rc = hip_status(launch_attention_local(a, stream));
  if (rc != SA_OK) return rc;
  return sparse_passes(plan, a, stream);
}

int sparse_attn_forward(const sa_params* p, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream,
                        hipStream_t side_stream, sa_plan** out) {
  if (out == nullptr) return SA_ERR_NULL_POINTER;
  *out = nullptr;
  if (v == nullptr || o == nullptr) return SA_ERR_NULL_POINTER;
  sa_plan* pl = nullptr;
  int rc = plan_create(p, q, k, workspace, workspace_bytes, &pl);
  if (rc != SA_OK) return rc;
  const AttnArgs a = attn_args(pl, q, k, v, o, lse);
  if (side_stream == stream) {  // one stream: plan, then prefill
    rc = plan_launch(pl, stream);
    if (rc == SA_OK) rc = hip_status(launch_attention_local(a, stream));
    if (rc == SA_OK) rc = sparse_passes(pl, a, stream);
  } else {
    // the local pass (which needs none of the plan's results) on the side
    // stream while the planner runs on `stream`; the sparse passes wait for
    // both
    hipEvent_t ready = nullptr, local_done = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ready, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&local_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ready, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side_stream, ready, 0);
    if (e == hipSuccess) e = launch_attention_local(a, side_stream);
    if (e == hipSuccess) e = hipEventRecord(local_done, side_stream);
    rc = hip_status(e);
    if (rc == SA_OK) rc = plan_launch(pl, stream);
    if (rc == SA_OK) rc = hip_status(hipStreamWaitEvent(stream, local_done, 0));
    if (rc == SA_OK) rc = sparse_passes(pl, a, stream);
    // released once the work recorded on them has completed
    if (ready != nullptr) (void)hipEventDestroy(ready);
    if (local_done != nullptr) (void)hipEventDestroy(local_done);
  }
  if (rc != SA_OK) {
    delete pl;
    return rc;
  }
  *out = pl;
  return SA_OK;
}

int sparse_attn_plan_set_max_threshold(sa_plan* plan, double theta) {
  if (plan == nullptr) return SA_ERR_NULL_POINTER;
  plan->max_theta = theta;
  plan->stops_valid = false;
  return SA_OK;
}

size_t sparse_attn_topk_scratch_bytes(const sa_plan* plan) {
  if (plan == nullptr) return 0;
  const PlanDims& d = plan->d;
  return topk_scratch_bytes(d.B, d.Hq, d.S, d.T);
}

int sparse_attn_plan_set_topk(sa_plan* plan, int32_t tiles, void* scratch,
                              size_t scratch_bytes, hipStream_t stream) {
  if (plan == nullptr) return SA_ERR_NULL_POINTER;
  if (tiles < 0) {  // back to the tau stop (or a budget)
    plan->topk = -1;
    plan->stops_valid = false;
    return SA_OK;
  }
  const PlanDims& d = plan->d;
  const size_t need = topk_scratch_bytes(d.B, d.Hq, d.S, d.T);
  if (need > 0 && scratch == nullptr) return SA_ERR_NULL_POINTER;
  if (scratch_bytes < need) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (reinterpret_cast<uintptr_t>(scratch) % 8 != 0) return SA_ERR_INVALID_ARG;
  TopkArgs a;
  a.q = static_cast<const uint16_t*>(plan->q);
  a.k = static_cast<const uint16_t*>(plan->k);
  a.pi_q = plan->at<int32_t>(plan->lay.pi_q);
  a.L = plan->at<int32_t>(plan->lay.L);
  a.scores = static_cast<int64_t*>(scratch);
  a.tmask = plan->at<uint32_t>(plan->lay.tmask);
  a.n_I = plan->at<int32_t>(plan->lay.n_I);
  a.list_len = (long long)d.list_len;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.S = d.S;
  a.T = d.T;
  a.G = d.G;
  a.K = tiles;
  // n_I now counts the selected tiles; leaving the mode rescans the stop
  // points
  plan->stops_valid = false;
  plan->topk = -1;
  const hipError_t e = launch_topk(a, stream);
  if (e != hipSuccess) return SA_ERR_HIP;
  plan->topk = tiles;
  return SA_OK;
}

int sparse_attn_plan_set_budget(sa_plan* plan, int32_t tiles) {
  if (plan == nullptr) return SA_ERR_NULL_POINTER;
  plan->budget = tiles < 0 ? -1 : tiles;
  plan->stops_valid = false;
  return SA_OK;
}

int sparse_attn_plan_set_tau(sa_plan* plan, double tau) {
  if (plan == nullptr) return SA_ERR_NULL_POINTER;
  if (!(tau >= 0.0) || std::isinf(tau)) return SA_ERR_INVALID_ARG;
  plan->p.tau = tau;
  plan->stops_valid = false;
  return SA_OK;
}

size_t sparse_attn_plan_export_bytes(const sa_plan* plan, int what) {
  if (plan == nullptr) return 0;
  const PlanDims& d = plan->d;
  const size_t nbg = (size_t)d.B * d.Hkv, nbh = (size_t)d.B * d.Hq;
  switch (what) {
    case SA_EXPORT_PI_K: return nbg * d.N * sizeof(int32_t);
    case SA_EXPORT_PI_Q: return nbh * d.N * sizeof(int32_t);
    case SA_EXPORT_L: return nbg * d.list_len * sizeof(int32_t);
    case SA_EXPORT_N_I: return nbh * (d.N / kBlock) * sizeof(int32_t);
    case SA_EXPORT_KEY_SCORE: return nbg * d.N * sizeof(int64_t);
    case SA_EXPORT_QUERY_SCORE: return nbh * d.N * sizeof(int64_t);
    case SA_EXPORT_CONTRAST: return nbg * d.T * kHeadDim * sizeof(int64_t);
    case SA_EXPORT_POOLED: return nbg * kHeadDim * sizeof(int64_t);
    case SA_EXPORT_TOPK_MASK:
      return nbh * (d.N / kBlock) * kMaskWords * sizeof(uint32_t);
    default: return 0;
  }
}

int sparse_attn_plan_export(const sa_plan* plan, int what, void* host_dst,
                            size_t bytes, hipStream_t stream) {
  if (plan == nullptr || host_dst == nullptr) return SA_ERR_NULL_POINTER;
  const size_t need = sparse_attn_plan_export_bytes(plan, what);
  if (need == 0 && what != SA_EXPORT_L) return SA_ERR_INVALID_ARG;
  if (bytes < need) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (need == 0) return SA_OK;
  size_t off = 0;
  switch (what) {
    case SA_EXPORT_PI_K: off = plan->lay.pi_k; break;
    case SA_EXPORT_PI_Q: off = plan->lay.pi_q; break;
    case SA_EXPORT_L: off = plan->lay.L; break;
    case SA_EXPORT_N_I: off = plan->lay.n_I; break;
    case SA_EXPORT_KEY_SCORE: off = plan->lay.vscore; break;
    case SA_EXPORT_QUERY_SCORE: off = plan->lay.u; break;
    case SA_EXPORT_CONTRAST: off = plan->lay.contrast; break;
    case SA_EXPORT_POOLED: off = plan->lay.pooled; break;
    case SA_EXPORT_TOPK_MASK: off = plan->lay.tmask; break;
  }
  hipError_t e = hipMemcpyAsync(host_dst, plan->ws + off, need,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e);
}

int sparse_attn_plan_set_kv_order(sa_plan* plan, const void* pi_k,
                                  hipStream_t stream) {
  if (plan == nullptr || pi_k == nullptr) return SA_ERR_NULL_POINTER;
  // a segment-local order's tiles must not mix segments: no injection
  if (segment_kv(plan->p)) return SA_ERR_INVALID_ARG;
  const size_t bytes = (size_t)plan->d.B * plan->d.Hkv * plan->d.N *
                       sizeof(int32_t);
  hipError_t e = hipMemcpyAsync(plan->ws + plan->lay.pi_k, pi_k, bytes,
                                hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return SA_ERR_HIP;
  plan->stops_valid = false;
  plan->topk = -1;  // the selections were made on the old lists
  const int rc = build_from_kv_order(plan, stream);
  return rc != SA_OK ? rc : run_stop_scan(plan, stream);
}

void sparse_attn_plan_destroy(sa_plan* plan) { delete plan; }

const char* sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SA_ERR_HIP: return "HIP runtime error";
    case SA_ERR_NULL_POINTER: return "null pointer";
    case SA_ERR_HOST_ALLOC: return "host allocation failed";
    default: return "unknown status";
  }
}

int sparse_attn_forward_static(const sa_params* p, const void* q,
                               const void* k, const void* v, void* o,
                               float* lse, hipStream_t stream) {
  const int st = validate(p);
  if (st != SA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return SA_ERR_NULL_POINTER;
  if (layout_of(dims_of(p)).total > SA_STATIC_SCRATCH_BYTES)
    return SA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  int rc = static_scratch(&ws);
  if (rc != SA_OK) return rc;
  // every array of the layout is written before it is read within this
  // call (the residuals are read only where this call's local pass wrote
  // them), so nothing carries over from an earlier call
  sa_plan pl;
  plan_fill(&pl, p, q, k, ws);
  rc = plan_launch(&pl, stream);
  if (rc != SA_OK) return rc;
  const AttnArgs a = attn_args(&pl, q, k, v, o, lse);
  rc = hip_status(launch_attention_local(a, stream));
  if (rc != SA_OK) return rc;
  return sparse_passes(&pl, a, stream);
}

}  // extern "C"
