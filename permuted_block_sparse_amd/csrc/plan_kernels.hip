// Importance estimator and index builder of permuted block-sparse prefill
// attention (S2O page, Summary: a segment-local query ordering and a global
// key/value ordering ranked by stripe-level mean pooling, kept as index
// arrays; no tensor is moved). Every score here is an exact integer built
// from the fixed-point images fx(x) = clamp(rint(256 x), -32768, 32767), so
// the orders do not depend on summation order and are bit-reproducible.
//
// All kernels are HBM-bound streaming passes (pooling, scoring), LDS sorts
// or index compaction; none is a dense contraction, so none uses MFMA.

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

// --------------------------------------------------------------------------
// Pooled group query: part[b, h, chunk, :] = sum of fx(q) over the chunk's
// rows. 16 lanes cover one 256-byte row with 16-byte loads (coalesced), 16
// rows per pass.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pool_q(const uint16_t* __restrict__ q,
                                                int64_t* __restrict__ part,
                                                int N, int nchunk) {
  __shared__ int32_t red[16][kHeadDim];
  const int blk = blockIdx.x;
  const int bh = blk / nchunk, ch = blk % nchunk;
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;
  const int row0 = ch * kPoolRows;
  const int rows = min(kPoolRows, N - row0);
  const uint16_t* base = q + ((size_t)bh * N + row0) * kHeadDim + c * 8;
  int32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0; r < rows; r += 16) {
    uint4 w = *reinterpret_cast<const uint4*>(base + (size_t)r * kHeadDim);
    int32_t f[8];
    fixed_point8(w, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i][tid];
    part[(size_t)blk * kHeadDim + tid] = s;
  }
}

// pooled[b, g, :] = sum over the G heads of group g and all chunks: one
// workgroup per (b, g), 8 slices of the G * nchunk partials per dimension,
// 8 independent loads in flight per thread, then a sum over the slices
// (integer: the order does not matter).
__global__ __launch_bounds__(1024) void k_pool_reduce(
    const int64_t* __restrict__ part, int64_t* __restrict__ pooled, int Hq,
    int Hkv, int nchunk) {
  __shared__ int64_t red[8][kHeadDim];
  const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
  const int d = threadIdx.x & (kHeadDim - 1), slice = threadIdx.x >> 7;
  const int n = G * nchunk;  // partials of the group, in (head, chunk) order
  const int64_t* p = part + ((size_t)(b * Hq + g * G) * nchunk) * kHeadDim + d;
  int64_t a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int i = slice;
  for (; i + 56 < n; i += 64) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += p[(size_t)(i + 8 * j) * kHeadDim];
  }
  for (; i < n; i += 8) a[0] += p[(size_t)i * kHeadDim];
  red[slice][d] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (slice == 0) {
    int64_t s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += red[j][d];
    pooled[(size_t)bg * kHeadDim + d] = s;
  }
}

// An int64 factor c of the stripe scores as c = lo + hi 2^32 with lo the
// signed low word: fx (|fx| <= 2^15) times c is then one 32 x 32 -> 64-bit
// multiply-add and one 24-bit one, exactly. The pooled query (|P| <= 2^40:
// G <= 256, N <= 2^17) and C_t (|C| <= 2^39) leave |hi| <= 2^8.
struct Split64 {
  int32_t lo, hi;
};
__device__ __forceinline__ Split64 split64(int64_t c) {
  Split64 r;
  r.lo = (int32_t)(uint32_t)(uint64_t)c;
  r.hi = (int32_t)((c - (int64_t)r.lo) >> 32);
  return r;
}
// sum over e of f[e] c[e], exact in int64
__device__ __forceinline__ int64_t dot8_split(const int32_t (&f)[8],
                                              const Split64 (&c)[8]) {
  int64_t lo = 0;
  int32_t hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo += (int64_t)f[e] * c[e].lo;
    hi += __mul24(f[e], c[e].hi);  // both within 24 bits
  }
  return lo + ((int64_t)hi << 32);
}

// --------------------------------------------------------------------------
// Key stripe score v_j = pooled . fx(k_j) (int64) and, on the same pass over
// K, the per-64-row column sums of fx(k) (int32; |sum| <= 64 * 2^15) and the
// workgroup's largest squared key norm (fp32; their maximum bounds the
// attention kernel's logits).
// --------------------------------------------------------------------------
// One workgroup covers kScoreRows = 16 passes of 16 rows (four 64-row key
// blocks), the shape of its loop and of its LDS reduction.
static_assert(kScoreRows == 16 * 16 && kScoreRows == 4 * kBlock,
              "k_key_score covers 16 passes of 16 rows per workgroup");
__global__ __launch_bounds__(256) void k_key_score(
    const uint16_t* __restrict__ k, const int64_t* __restrict__ pooled,
    int64_t* __restrict__ vscore, int32_t* __restrict__ blocksum,
    float* __restrict__ kpart, int N, int nwg) {
  __shared__ int32_t red[4][16][kHeadDim];
  __shared__ float wmax[4];
  const int bg = blockIdx.x / nwg, w = blockIdx.x % nwg;
  const int tid = threadIdx.x, c = tid & 15, rr = tid >> 4;
  const int row0 = w * kScoreRows;
  const int rows = min(kScoreRows, N - row0);  // a multiple of 64
  Split64 p8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    p8[e] = split64(pooled[(size_t)bg * kHeadDim + c * 8 + e]);
  const uint16_t* base = k + ((size_t)bg * N + row0) * kHeadDim + c * 8;
  int32_t bs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float kn = 0.f;  // largest |k|^2 of this thread's rows
  for (int p = 0; p < 16; ++p) {
    const int r = rr + 16 * p;
    if (p * 16 < rows) {  // uniform over the workgroup
      uint4 wv = *reinterpret_cast<const uint4*>(base + (size_t)r * kHeadDim);
      int32_t f[8];
      fixed_point8(wv, f);
      int64_t dot = dot8_split(f, p8);
#pragma unroll
      for (int e = 0; e < 8; ++e) bs[e] += f[e];
      dot = sum16_i64(dot);
      if (c == 0) vscore[(size_t)bg * N + row0 + r] = dot;
      const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(wd[e] << 16);
        const float hi = __uint_as_float(wd[e] & 0xffff0000u);
        sq = fmaf(lo, lo, sq);
        sq = fmaf(hi, hi, sq);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o);
      kn = fmaxf(kn, sq);
    }
    if ((p & 3) == 3) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red[p >> 2][rr][c * 8 + e] = bs[e];
        bs[e] = 0;
      }
    }
  }
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) kn = fmaxf(kn, __shfl_xor(kn, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = kn;
  __syncthreads();
  if (tid == 0)
    kpart[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int nblk = rows / kBlock;
  for (int i = tid; i < 4 * kHeadDim; i += 256) {
    const int bl = i / kHeadDim, d = i % kHeadDim;
    if (bl < nblk) {
      int32_t s = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) s += red[bl][j][d];
      blocksum[((size_t)bg * (N / kBlock) + row0 / kBlock + bl) * kHeadDim + d] =
          s;
    }
  }
}

// segsum[b, g, t, :] = sum of fx(k) over segment t; the t = 0 workgroup
// also reduces the key-score workgroups' largest |k|^2 to kmax2[b, g].
__global__ __launch_bounds__(128) void k_segment_sum(
    const int32_t* __restrict__ blocksum, int64_t* __restrict__ segsum,
    const float* __restrict__ kpart, float* __restrict__ kmax2, int N, int S,
    int T, int nwg) {
  const int bgt = blockIdx.x, bg = bgt / T, t = bgt % T, d = threadIdx.x;
  if (t == 0) {  // uniform over the workgroup
    __shared__ float wmax[2];
    float x = 0.f;
    for (int i = d; i < nwg; i += 128) x = fmaxf(x, kpart[(size_t)bg * nwg + i]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    if ((d & 63) == 0) wmax[d >> 6] = x;
    __syncthreads();
    if (d == 0) kmax2[bg] = fmaxf(wmax[0], wmax[1]);
  }
  const int nb = S / kBlock;
  const int32_t* p =
      blocksum + ((size_t)bg * (N / kBlock) + (size_t)t * nb) * kHeadDim + d;
  int64_t s = 0;
  for (int i = 0; i < nb; ++i) s += p[(size_t)i * kHeadDim];
  segsum[(size_t)bgt * kHeadDim + d] = s;
}

// --------------------------------------------------------------------------
// Contrast vectors C_t = t S * sum_{j in L_t[0:64]} fx(k_j)
//                       - 64 * sum_{j < t S} fx(k_j)     (t = 0: zero).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_contrast(
    const uint16_t* __restrict__ k, const int32_t* __restrict__ L,
    const int64_t* __restrict__ segsum, int64_t* __restrict__ contrast, int N,
    int S, int T, long long list_len) {
  const int bgt = blockIdx.x, bg = bgt / T, t = bgt % T, d = threadIdx.x;
  int64_t c = 0;
  if (t > 0) {
    const int32_t* Lt = L + (size_t)bg * list_len + (size_t)S * t * (t - 1) / 2;
    const uint16_t* kb = k + (size_t)bg * N * kHeadDim + d;
    int64_t top = 0;
    for (int r = 0; r < kBlock; ++r) {
      const int key = min(max(Lt[r], 0), N - 1);  // memory-safe for any L
      top += fixed_point(kb[(size_t)key * kHeadDim]);
    }
    int64_t pre = 0;
    for (int s2 = 0; s2 < t; ++s2)
      pre += segsum[((size_t)bg * T + s2) * kHeadDim + d];
    c = (int64_t)t * S * top - (int64_t)kBlock * pre;
  }
  contrast[(size_t)bgt * kHeadDim + d] = c;
}

// Query stripe score u_i = fx(q_i) . C_seg(i) (C_0 = 0, so u = 0 there).
// int64 sum of the 16 lanes of each aligned 16-lane row, in lane 15 of the
// row (DPP row shifts; integer addition, so the order does not matter).
__device__ __forceinline__ int64_t row16_sum_i64(int64_t v) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) {
    const int lo = (int)(uint32_t)(uint64_t)v;
    const int hi = (int)(uint32_t)((uint64_t)v >> 32);
    // row_shr:sh (0x110 + sh); lanes below the shift read 0
    const int slo = sh == 1 ? __builtin_amdgcn_update_dpp(0, lo, 0x111, 0xF, 0xF, false)
                  : sh == 2 ? __builtin_amdgcn_update_dpp(0, lo, 0x112, 0xF, 0xF, false)
                  : sh == 4 ? __builtin_amdgcn_update_dpp(0, lo, 0x114, 0xF, 0xF, false)
                            : __builtin_amdgcn_update_dpp(0, lo, 0x118, 0xF, 0xF, false);
    const int shi = sh == 1 ? __builtin_amdgcn_update_dpp(0, hi, 0x111, 0xF, 0xF, false)
                  : sh == 2 ? __builtin_amdgcn_update_dpp(0, hi, 0x112, 0xF, 0xF, false)
                  : sh == 4 ? __builtin_amdgcn_update_dpp(0, hi, 0x114, 0xF, 0xF, false)
                            : __builtin_amdgcn_update_dpp(0, hi, 0x118, 0xF, 0xF, false);
    v += (int64_t)(((uint64_t)(uint32_t)shi << 32) | (uint32_t)slo);
  }
  return v;
}

__global__ __launch_bounds__(256) void k_query_score(
    const uint16_t* __restrict__ q, const int64_t* __restrict__ contrast,
    int64_t* __restrict__ u, int Hq, int Hkv, int N, int S, int T, int nwg) {
  const int bh = blockIdx.x / nwg, w = blockIdx.x % nwg;
  const int b = bh / Hq, h = bh % Hq, G = Hq / Hkv;
  const int bg = b * Hkv + h / G;
  const int tid = threadIdx.x, c = tid & 15, rr = tid >> 4;
  const int row0 = w * kScoreRows;
  const int rows = min(kScoreRows, N - row0);
  const uint16_t* base = q + ((size_t)bh * N + row0) * kHeadDim + c * 8;
  // this lane's 8 entries of C_t, reloaded when the segment changes
  int t_loaded = -1;
  Split64 cv[8];
  for (int p = 0; p * 16 < rows; ++p) {
    const int r = rr + 16 * p;
    const int t = (row0 + r) / S;
    if (t != t_loaded) {
      const int64_t* src = contrast + ((size_t)bg * T + t) * kHeadDim + c * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) cv[e] = split64(src[e]);
      t_loaded = t;
    }
    uint4 wv = *reinterpret_cast<const uint4*>(base + (size_t)r * kHeadDim);
    int32_t f[8];
    fixed_point8(wv, f);
    int64_t dot = dot8_split(f, cv);
    dot = row16_sum_i64(dot);
    if (c == 15) u[(size_t)bh * N + row0 + r] = dot;
  }
}

// --------------------------------------------------------------------------
// Segmented argsort by (score descending, index ascending). A workgroup
// sorts a chunk of up to 4096 elements: each thread sorts E consecutive
// elements in registers (a bitonic network), then log2(256) merge rounds in
// LDS double the sorted runs, each thread finding its E outputs of a round
// by a merge-path search. Longer segments are finished by merge passes over
// global memory. The composite keys are unique, so the result does not
// depend on the algorithm.
// --------------------------------------------------------------------------
__device__ __forceinline__ void cmp_swap(uint64_t* key, int32_t* idx, int i,
                                         int l, bool up) {
  uint64_t ka = key[i], kb = key[l];
  int32_t ia = idx[i], ib = idx[l];
  const bool gt = pair_less(kb, ib, ka, ia);
  if (gt == up) {
    key[i] = kb; key[l] = ka;
    idx[i] = ib; idx[l] = ia;
  }
}

// Merge-path split of diagonal x of two sorted runs A (la) and B (lb): the
// number of A elements among the first x outputs.
__device__ __forceinline__ int merge_split(const uint64_t* KA, const int32_t* IA,
                                           int la, const uint64_t* KB,
                                           const int32_t* IB, int lb, int x) {
  int lo = max(0, x - lb), hi = min(x, la);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pair_less(KA[mid], IA[mid], KB[x - 1 - mid], IB[x - 1 - mid]))
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// n outputs of the merge of A and B starting at A[i], B[j] (n <= the
// elements left), into registers.
template <int E>
__device__ __forceinline__ void merge_run(const uint64_t* KA, const int32_t* IA,
                                          int la, const uint64_t* KB,
                                          const int32_t* IB, int lb, int i,
                                          int j, uint64_t (&rk)[E],
                                          int32_t (&ri)[E]) {
  // heads of both runs; an exhausted (or empty) run's head is a clamped,
  // in-bounds read that the j >= lb / i < la tests never use
  auto ca = [&](int v) { return max(min(v, la - 1), 0); };
  auto cb = [&](int v) { return max(min(v, lb - 1), 0); };
  uint64_t ha = KA[ca(i)], hb = KB[cb(j)];
  int32_t hia = IA[ca(i)], hib = IB[cb(j)];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool ta = j >= lb || (i < la && pair_less(ha, hia, hb, hib));
    rk[e] = ta ? ha : hb;
    ri[e] = ta ? hia : hib;
    if (ta) {
      ++i;
      ha = KA[ca(i)];
      hia = IA[ca(i)];
    } else {
      ++j;
      hb = KB[cb(j)];
      hib = IB[cb(j)];
    }
  }
}

template <int E>
__global__ __launch_bounds__(256) void k_chunk_sort(
    const int64_t* __restrict__ score, int seglen, int rowlen, int chunk,
    int nch, uint64_t* __restrict__ okey, int32_t* __restrict__ oidx,
    int32_t* __restrict__ out) {
  constexpr int n = 256 * E;  // >= the chunk; the rest is padding
  __shared__ uint64_t key[n];
  __shared__ int32_t idx[n];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x / nch, ch = blockIdx.x % nch;
  const int start = ch * chunk;
  const int cnt = min(chunk, seglen - start);
  const size_t gbase = (size_t)seg * seglen + start;
  for (int i = tid; i < n; i += 256) {
    if (i < cnt) {
      key[i] = desc_key(score[gbase + i]);
      idx[i] = (int32_t)((gbase + i) % (size_t)rowlen);
    } else {  // after every real element
      key[i] = ~0ull;
      idx[i] = 0x7fffffff;
    }
  }
  __syncthreads();
  // this thread's E elements, sorted in registers
  uint64_t rk[E];
  int32_t ri[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    rk[e] = key[tid * E + e];
    ri[e] = idx[tid * E + e];
  }
#pragma unroll
  for (int kk = 2; kk <= E; kk <<= 1)
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int l = i ^ j;
        if (l > i && pair_less(rk[l], ri[l], rk[i], ri[i]) == ((i & kk) == 0)) {
          const uint64_t tk = rk[i]; rk[i] = rk[l]; rk[l] = tk;
          const int32_t ti = ri[i]; ri[i] = ri[l]; ri[l] = ti;
        }
      }
  // merge rounds: runs of w become runs of 2 w (every run is full: n is a
  // power of two)
  for (int w = E; w < n; w <<= 1) {
    __syncthreads();  // everyone has read the previous runs
#pragma unroll
    for (int e = 0; e < E; ++e) {
      key[tid * E + e] = rk[e];
      idx[tid * E + e] = ri[e];
    }
    __syncthreads();
    const int o = tid * E;
    const int a0 = o & ~(2 * w - 1);
    const uint64_t* KA = key + a0;
    const int32_t* IA = idx + a0;
    const int x = o - a0;
    const int i = merge_split(KA, IA, w, KA + w, IA + w, w, x);
    merge_run<E>(KA, IA, w, KA + w, IA + w, w, i, x - i, rk, ri);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[tid * E + e] = rk[e];
    idx[tid * E + e] = ri[e];
  }
  __syncthreads();
  for (int i = tid; i < cnt; i += 256) {
    if (out != nullptr) {
      out[gbase + i] = idx[i];
    } else {
      okey[gbase + i] = key[i];
      oidx[gbase + i] = idx[i];
    }
  }
}

// One merge pass over global memory: runs of `width` (a multiple of
// kMergeTile / 2) become runs of 2 width. Workgroup p of a segment emits its
// outputs [kMergeTile p, kMergeTile (p + 1)): a k-ary merge-path search (128
// candidates per round and per end) finds where the range starts and ends in
// the two runs, both input windows go to LDS, each thread merges 8 outputs
// from there, and the outputs leave in coalesced rows.
constexpr int kMergeTile = 2048;

__global__ __launch_bounds__(256) void k_merge_pass(
    const uint64_t* __restrict__ ikey, const int32_t* __restrict__ iidx,
    uint64_t* __restrict__ okey, int32_t* __restrict__ oidx,
    int32_t* __restrict__ out, int seglen, int width, int tiles_per_seg) {
  __shared__ uint64_t sk[kMergeTile];
  __shared__ int32_t si[kMergeTile];
  __shared__ int s_lo[2], s_hi[2], s_cnt[4];
  const int tid = threadIdx.x, hsel = tid >> 7, t = tid & 127;
  const int seg = blockIdx.x / tiles_per_seg;
  const int o0 = (blockIdx.x % tiles_per_seg) * kMergeTile;
  const int o1 = min(o0 + kMergeTile, seglen);
  const int a0 = (o0 / (2 * width)) * 2 * width;  // o1 - 1 is in this pair
  const int a1 = min(a0 + width, seglen), b1 = min(a0 + 2 * width, seglen);
  const int la = a1 - a0, lb = b1 - a1;
  const size_t base = (size_t)seg * seglen;
  const uint64_t* KA = ikey + base + a0;
  const int32_t* IA = iidx + base + a0;
  const uint64_t* KB = ikey + base + a1;
  const int32_t* IB = iidx + base + a1;

  // splits of diagonals o0 - a0 (threads 0..127) and o1 - a0 (128..255);
  // each round samples 128 points of [lo, hi), where the predicate "A[m]
  // comes before B[x - 1 - m]" is true below the split and false above
  const int x = (hsel ? o1 : o0) - a0;
  if (t == 0) {
    s_lo[hsel] = max(0, x - lb);
    s_hi[hsel] = min(x, la);
  }
  __syncthreads();
  for (;;) {
    const int lo = s_lo[hsel], hi = s_hi[hsel];
    const int R = hi - lo;
    const int m = lo + (int)(((long long)R * t) >> 7);  // in [lo, hi) if R > 0
    const bool pr =
        R > 0 && pair_less(KA[m], IA[m], KB[x - 1 - m], IB[x - 1 - m]);
    const unsigned long long bal = __ballot(pr);
    if ((tid & 63) == 0) s_cnt[tid >> 6] = __popcll(bal);
    __syncthreads();
    const int c = s_cnt[2 * hsel] + s_cnt[2 * hsel + 1];  // true prefix
    __syncthreads();  // every thread has read lo, hi and the counts
    if (R > 0) {
      if (t == c - 1) s_lo[hsel] = m + 1;
      if (t == c) s_hi[hsel] = m;
    }
    __syncthreads();
    if (s_lo[0] == s_hi[0] && s_lo[1] == s_hi[1]) break;  // uniform
  }
  const int ia0 = s_lo[0], ia1 = s_lo[1];
  const int ib0 = (o0 - a0) - ia0, ib1 = (o1 - a0) - ia1;
  const int na = ia1 - ia0, nb = ib1 - ib0;  // na + nb = o1 - o0
  for (int i = tid; i < na; i += 256) {
    sk[i] = KA[ia0 + i];
    si[i] = IA[ia0 + i];
  }
  for (int i = tid; i < nb; i += 256) {
    sk[na + i] = KB[ib0 + i];
    si[na + i] = IB[ib0 + i];
  }
  __syncthreads();
  uint64_t rk[8];
  int32_t ri[8];
  const int y = 8 * tid;
  const int n_out = o1 - o0;
  if (y < n_out) {
    const int i = merge_split(sk, si, na, sk + na, si + na, nb, y);
    merge_run<8>(sk, si, na, sk + na, si + na, nb, i, y - i, rk, ri);
  }
  __syncthreads();
  if (y < n_out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (y + e < n_out) {
        sk[y + e] = rk[e];
        si[y + e] = ri[e];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < n_out; i += 256) {
    if (out != nullptr) {
      out[base + o0 + i] = si[i];
    } else {
      okey[base + o0 + i] = sk[i];
      oidx[base + o0 + i] = si[i];
    }
  }
}

__global__ void k_iota(int32_t* __restrict__ out, size_t n, int rowlen) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = (int32_t)(i % (size_t)rowlen);
}

// --------------------------------------------------------------------------
// Causal restriction: L_t = pi_K without keys >= t S, order kept, t >= 1.
// cnt[bg, ch, t] = #{entries of chunk ch with segment < t};
// cum[bg, ch, t] = sum of cnt over earlier chunks (the write offset).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_restrict_count(
    const int32_t* __restrict__ pi_k, int32_t* __restrict__ cnt, int N, int S,
    int T, int nrc) {
  extern __shared__ int32_t hist[];  // T + 1 entries
  const int bg = blockIdx.x / nrc, ch = blockIdx.x % nrc;
  for (int i = threadIdx.x; i <= T; i += 256) hist[i] = 0;
  __syncthreads();
  const int start = ch * kRestrictChunk;
  const int n = min(kRestrictChunk, N - start);
  const int32_t* p = pi_k + (size_t)bg * N + start;
  for (int i = threadIdx.x; i < n; i += 256)
    atomicAdd(&hist[min(max(p[i] / S, 0), T - 1)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive prefix over segments, T <= 2048
    int run = 0;
    for (int s = 0; s < T; ++s) {
      const int v = hist[s];
      hist[s] = run;
      run += v;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += 256)
    cnt[((size_t)bg * nrc + ch) * T + t] = hist[t];
}

__global__ __launch_bounds__(256) void k_restrict_scan(
    const int32_t* __restrict__ cnt, int32_t* __restrict__ cum, int T,
    int nrc) {
  const int bg = blockIdx.x;
  for (int t = threadIdx.x; t < T; t += 256) {
    int run = 0;
    for (int ch = 0; ch < nrc; ++ch) {
      const size_t i = ((size_t)bg * nrc + ch) * T + t;
      cum[i] = run;
      run += cnt[i];
    }
  }
}

// Exclusive scan of one int per thread over a 256-thread workgroup.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum,
                                                    int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wid; ++w) before += wsum[w];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + x - v;
}

// One workgroup per (b, g, chunk, part): the chunk's entries go to the lists
// L_t with t = 1 + part, 1 + part + split, ... (interleaved, so the parts
// write about the same amount). Per list, the chunk's surviving entries are
// compacted in LDS and leave as one contiguous run.
__global__ __launch_bounds__(256) void k_restrict_write(
    const int32_t* __restrict__ pi_k, const int32_t* __restrict__ cum,
    int32_t* __restrict__ L, int N, int S, int T, int nrc, int split,
    long long list_len) {
  __shared__ int wsum[4];
  __shared__ int32_t buf[kRestrictChunk];
  const int part = blockIdx.x % split, bgc = blockIdx.x / split;
  const int bg = bgc / nrc, ch = bgc % nrc;
  const int start = ch * kRestrictChunk;
  const int n = min(kRestrictChunk, N - start);
  constexpr int kPer = kRestrictChunk / 256;
  int32_t keyv[kPer];
  int32_t segv[kPer];
  const int32_t* p = pi_k + (size_t)bg * N + start;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = threadIdx.x * kPer + e;
    keyv[e] = i < n ? p[i] : 0;
    segv[e] = i < n ? keyv[e] / S : 0x7fffffff;
  }
  int32_t* Lbg = L + (size_t)bg * list_len;
  for (int t = 1 + part; t < T; t += split) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) c += segv[e] < t;
    int total;
    int pos = block_exclusive_scan(c, wsum, total);  // total <= n
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (segv[e] < t) buf[pos++] = keyv[e];
    }
    __syncthreads();
    const int base = cum[((size_t)bg * nrc + ch) * T + t];
    int32_t* Lt = Lbg + (size_t)S * t * (t - 1) / 2;
    const int cap = t * S;  // |L_t|; only exceeded if pi_K is no permutation
    for (int i = threadIdx.x; i < total; i += 256)
      if (base + i < cap) Lt[base + i] = buf[i];
    __syncthreads();  // buf is refilled for the next list
  }
}

// --------------------------------------------------------------------------
// Segment-local key order (the PBS-Attn page's permutation inside causal
// segments): pi_K sorts the keys of each segment by v; its 64-key chunks are
// the tiles; segment t visits the tiles of segments 0 .. t - 1 by tile score
// (the sum of v over the tile, exact int64) descending, ties by tile index.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tile_score(
    const int64_t* __restrict__ v, const int32_t* __restrict__ pi_k,
    int64_t* __restrict__ tscore, int N, long long ntiles_total) {
  // one wave per tile, one key per lane
  const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles_total) return;
  const int lane = threadIdx.x & 63;
  const long long bg = tile / (N / 64);
  const int key = min(max(pi_k[tile * 64 + lane], 0), N - 1);
  int64_t s = v[bg * N + key];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += shfl_xor_i64(s, o);
  if (lane == 0) tscore[tile] = s;
}

__global__ __launch_bounds__(256) void k_segment_tiles(
    const int64_t* __restrict__ tscore, const int32_t* __restrict__ pi_k,
    int32_t* __restrict__ L, int N, int S, int T, long long list_len) {
  __shared__ uint64_t key[kMaxTiles];
  __shared__ int32_t idx[kMaxTiles];
  const int t = 1 + blockIdx.x % (T - 1);
  const long long bg = blockIdx.x / (T - 1);
  const int nt = t * (S / 64);  // tiles of segments 0 .. t - 1
  int np2 = 1;
  while (np2 < nt) np2 <<= 1;
  const int64_t* ts = tscore + bg * (N / 64);
  for (int i = threadIdx.x; i < np2; i += 256) {
    if (i < nt) {
      key[i] = desc_key(ts[i]);
      idx[i] = i;
    } else {
      key[i] = ~0ull;
      idx[i] = 0x7fffffff;
    }
  }
  __syncthreads();
  for (int kk = 2; kk <= np2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int p = threadIdx.x; p < (np2 >> 1); p += 256) {
        // j is a power of two: i = 2 j (p / j) + p % j
        const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
        cmp_swap(key, idx, i, i + j, (i & kk) == 0);
      }
      __syncthreads();
    }
  }
  int32_t* Lt = L + bg * list_len + (long long)S * t * (t - 1) / 2;
  const int32_t* pk = pi_k + bg * N;
  for (int i = threadIdx.x; i < nt * 64; i += 256)
    Lt[i] = pk[idx[i >> 6] * 64 + (i & 63)];
}

// --------------------------------------------------------------------------
// Launchers
// --------------------------------------------------------------------------
hipError_t launch_pool_q(const PlanDims& d, const uint16_t* q, int64_t* part,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_pool_q, dim3(d.B * d.Hq * d.n_pool_chunks), dim3(256), 0,
                     s, q, part, d.N, d.n_pool_chunks);
  return hipGetLastError();
}

hipError_t launch_pool_reduce(const PlanDims& d, const int64_t* part,
                              int64_t* pooled, hipStream_t s) {
  hipLaunchKernelGGL(k_pool_reduce, dim3(d.B * d.Hkv), dim3(8 * kHeadDim), 0,
                     s, part, pooled, d.Hq, d.Hkv, d.n_pool_chunks);
  return hipGetLastError();
}

hipError_t launch_key_score(const PlanDims& d, const uint16_t* k,
                            const int64_t* pooled, int64_t* vscore,
                            int32_t* blocksum, float* kpart, hipStream_t s) {
  hipLaunchKernelGGL(k_key_score, dim3(d.B * d.Hkv * d.n_score_wg), dim3(256),
                     0, s, k, pooled, vscore, blocksum, kpart, d.N,
                     d.n_score_wg);
  return hipGetLastError();
}

hipError_t launch_segment_sum(const PlanDims& d, const int32_t* blocksum,
                              int64_t* segsum, const float* kpart,
                              float* kmax2, hipStream_t s) {
  hipLaunchKernelGGL(k_segment_sum, dim3(d.B * d.Hkv * d.T), dim3(kHeadDim), 0,
                     s, blocksum, segsum, kpart, kmax2, d.N, d.S, d.T,
                     d.n_score_wg);
  return hipGetLastError();
}

hipError_t launch_contrast(const PlanDims& d, const uint16_t* k,
                           const int32_t* L, const int64_t* segsum,
                           int64_t* contrast, hipStream_t s) {
  hipLaunchKernelGGL(k_contrast, dim3(d.B * d.Hkv * d.T), dim3(kHeadDim), 0, s,
                     k, L, segsum, contrast, d.N, d.S, d.T,
                     (long long)d.list_len);
  return hipGetLastError();
}

hipError_t launch_query_score(const PlanDims& d, const uint16_t* q,
                              const int64_t* contrast, int64_t* u,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_query_score, dim3(d.B * d.Hq * d.n_score_wg), dim3(256),
                     0, s, q, contrast, u, d.Hq, d.Hkv, d.N, d.S, d.T,
                     d.n_score_wg);
  return hipGetLastError();
}

hipError_t launch_segmented_argsort(const int64_t* score, int n_seg,
                                    int seglen, int rowlen, uint64_t* key_a,
                                    int32_t* idx_a, uint64_t* key_b,
                                    int32_t* idx_b, int32_t* out,
                                    hipStream_t s) {
  const int chunk = seglen < kSortChunk ? seglen : kSortChunk;
  const int nch = (seglen + chunk - 1) / chunk;
  int np2 = 256;  // 256 threads x E elements, E a power of two <= 16
  while (np2 < chunk) np2 <<= 1;
  const bool single = nch == 1;
  int32_t* o1 = single ? out : nullptr;
  const dim3 g(n_seg * nch), b(256);
  switch (np2) {
    case 256: hipLaunchKernelGGL(k_chunk_sort<1>, g, b, 0, s, score, seglen, rowlen, chunk, nch, key_a, idx_a, o1); break;
    case 512: hipLaunchKernelGGL(k_chunk_sort<2>, g, b, 0, s, score, seglen, rowlen, chunk, nch, key_a, idx_a, o1); break;
    case 1024: hipLaunchKernelGGL(k_chunk_sort<4>, g, b, 0, s, score, seglen, rowlen, chunk, nch, key_a, idx_a, o1); break;
    case 2048: hipLaunchKernelGGL(k_chunk_sort<8>, g, b, 0, s, score, seglen, rowlen, chunk, nch, key_a, idx_a, o1); break;
    default: hipLaunchKernelGGL(k_chunk_sort<16>, g, b, 0, s, score, seglen, rowlen, chunk, nch, key_a, idx_a, o1); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || single) return e;
  // merge passes: widths chunk, 2 chunk, ... (multiples of kMergeTile / 2)
  const int tiles = (seglen + kMergeTile - 1) / kMergeTile;
  uint64_t* ki = key_a; int32_t* ii = idx_a;
  uint64_t* ko = key_b; int32_t* io = idx_b;
  for (int width = chunk; width < seglen; width *= 2) {
    const bool last = 2 * width >= seglen;
    hipLaunchKernelGGL(k_merge_pass, dim3(n_seg * tiles), dim3(256), 0, s, ki,
                       ii, ko, io, last ? out : nullptr, seglen, width, tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint64_t* tk = ki; ki = ko; ko = tk;
    int32_t* ti = ii; ii = io; io = ti;
  }
  return hipSuccess;
}

hipError_t launch_iota(int32_t* out, size_t n, int rowlen, hipStream_t s) {
  const int grid = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  hipLaunchKernelGGL(k_iota, dim3(grid), dim3(256), 0, s, out, n, rowlen);
  return hipGetLastError();
}

hipError_t launch_restrict(const PlanDims& d, const int32_t* pi_k,
                           int32_t* cnt, int32_t* cum, int32_t* L,
                           hipStream_t s) {
  if (d.T < 2) return hipSuccess;
  const int nbg = d.B * d.Hkv;
  hipLaunchKernelGGL(k_restrict_count, dim3(nbg * d.n_restrict_chunks),
                     dim3(256), (d.T + 1) * sizeof(int32_t), s, pi_k, cnt, d.N,
                     d.S, d.T, d.n_restrict_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_restrict_scan, dim3(nbg), dim3(256), 0, s, cnt, cum,
                     d.T, d.n_restrict_chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int split = d.T - 1 < kRestrictSplit ? d.T - 1 : kRestrictSplit;
  hipLaunchKernelGGL(k_restrict_write,
                     dim3(nbg * d.n_restrict_chunks * split), dim3(256), 0, s,
                     pi_k, cum, L, d.N, d.S, d.T, d.n_restrict_chunks, split,
                     (long long)d.list_len);
  return hipGetLastError();
}

hipError_t launch_segment_tiles(const PlanDims& d, const int64_t* v,
                                const int32_t* pi_k, int64_t* tscore,
                                int32_t* L, hipStream_t s) {
  if (d.T < 2) return hipSuccess;
  const long long nbg = (long long)d.B * d.Hkv;
  const long long ntiles = nbg * (d.N / 64);
  hipLaunchKernelGGL(k_tile_score, dim3((unsigned)((ntiles + 3) / 4)),
                     dim3(256), 0, s, v, pi_k, tscore, d.N, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_segment_tiles, dim3((unsigned)(nbg * (d.T - 1))),
                     dim3(256), 0, s, tscore, pi_k, L, d.N, d.S, d.T,
                     (long long)d.list_len);
  return hipGetLastError();
}

}  // namespace sa
