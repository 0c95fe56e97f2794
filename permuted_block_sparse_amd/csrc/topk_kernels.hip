// Per-block Top-K tile selection from mean-pooled centroids, the alternative
// to the tau stop that the AB-Sparse page describes (block-sparse workflow,
// the paragraph around its Figure 2 with the footnote on mean pooling):
// every key block is scored by the product of the query with the block's
// centroid (its mean key) and the best K blocks are attended. Here the
// query side is a query block of pi_Q (its mean query), the key blocks are
// the tiles of L_t, and both means are taken in the fixed-point images of
// the orders, so the scores are exact integers:
//   r(I, k) = (sum of fx(q) over block I's 64 rows) . (sum of fx(k) over
//             tile k's 64 keys),
// |each sum| <= 64 * 2^15 = 2^21, |r| <= 128 * 2^42 = 2^49. Both sums are
// exact in fp32 and every product and partial sum of the contraction is an
// integer below 2^53, so the scores are computed exactly by the fp64 MFMA
// (v_mfma_f64_16x16x4f64) as one GEMM per group: [blocks x 128] times
// [128 x tiles of L_t].
//
//   k_topk_scores : per (b, KV head, segment t >= 1) and up to 128 query
//                   blocks of its G heads: the blocks' sums, then the tiles
//                   of L_t 32 at a time (gathered key rows -> sums in LDS ->
//                   MFMA), scores to a scratch array, int64;
//   k_topk_select : one wave per block: the min(K, t S / 64) tiles of
//                   highest score, ties by smaller position in L_t (an exact
//                   radix select on unique 62-bit keys), as a bitmask over
//                   the positions of L_t, and n_I = their count.

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kTkBlocks = 128;  // query blocks per scoring workgroup
constexpr int kTkTiles = 32;    // tiles of L_t per scoring step
constexpr int kTkStride = 132;  // LDS row stride (floats) of the sums
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Sum of fx over the 64 rows `row_of_lane` names (row r held by lane r) of a
// [*, 128] bf16 matrix, exact (int32): lane l adds 16-byte chunk l % 16 of
// rows l / 16, l / 16 + 4, ..., then the four row groups are added across
// lanes. Lanes 0..15 return dims 8 (l % 16) .. + 7.
static __device__ __forceinline__ void fx_sum_rows64(const uint16_t* base,
                                                     int row_of_lane, int lane,
                                                     int32_t (&s)[8]) {
  const int c = lane & 15, rg = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = __shfl(row_of_lane, rg + 4 * (8 * h + j));
      w[j] = *reinterpret_cast<const uint4*>(base + (size_t)row * kHeadDim +
                                             8 * c);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int32_t f[8];
      fixed_point8(w[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] += __shfl_xor(s[e], 16);
    s[e] += __shfl_xor(s[e], 32);
  }
}

// Offset of block I's scores (one per tile of L_t) in the scratch of one
// (b, h): blocks of segment t hold t * bps scores each, segments in order.
__device__ __forceinline__ long long topk_score_offset(int t, int i_in_seg,
                                                       int bps) {
  return (long long)bps * bps * t * (t - 1) / 2 + (long long)i_in_seg * t * bps;
}

__global__ __launch_bounds__(512) void k_topk_scores(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[kTkBlocks][kTkStride];
  __shared__ __attribute__((aligned(16))) float ks[kTkTiles][kTkStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bps = a.S / kBlock, per_group = a.G * bps;
  const int n_chunk = (per_group + kTkBlocks - 1) / kTkBlocks;
  const int BH = a.B * a.Hkv;
  // segments t = T-1 .. 1 (the longest first)
  const int p = blockIdx.x;
  const int t = a.T - 1 - p / (n_chunk * BH);
  const int rem = p % (n_chunk * BH);
  const int bg = rem / n_chunk, chunk = rem % n_chunk;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int ntl = t * bps;
  const long long per_bh = (long long)bps * bps * a.T * (a.T - 1) / 2;

  // block sums: wave w sums blocks 16 w .. 16 w + 15 of the chunk
  for (int jj = 0; jj < 16; ++jj) {
    const int j = 16 * wave + jj;
    const int e = chunk * kTkBlocks + j;
    int32_t s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (e < per_group) {  // wave-uniform
      const int h = g * a.G + e % a.G, I = t * bps + e / a.G;
      const long long bh = (long long)b * a.Hq + h;
      const int row = min(max(a.pi_q[bh * a.N + (long long)I * kBlock + lane],
                              0), a.N - 1);
      fx_sum_rows64(a.q + bh * (long long)a.N * kHeadDim, row, lane, s);
    }
    if (lane < 16) {
      float4* dst = reinterpret_cast<float4*>(&qs[j][8 * lane]);
      dst[0] = make_float4((float)s[0], (float)s[1], (float)s[2], (float)s[3]);
      dst[1] = make_float4((float)s[4], (float)s[5], (float)s[6], (float)s[7]);
    }
  }
  __syncthreads();
  // the wave's A operands for the whole run: lane l holds block
  // 16 w + l % 16, dims 4 s + l / 16 (s = 0..31); B operands: lane l holds
  // tile 16 c + l % 16, dims 4 s + l / 16
  double aq[32];
#pragma unroll
  for (int s = 0; s < 32; ++s)
    aq[s] = (double)qs[16 * wave + (lane & 15)][4 * s + (lane >> 4)];

  const uint16_t* kbase = a.k + (long long)bg * a.N * kHeadDim;
  const int32_t* Lt =
      a.L + (long long)bg * a.list_len + (long long)a.S * t * (t - 1) / 2;
  for (int k0 = 0; k0 < ntl; k0 += kTkTiles) {
    const int cnt = min(kTkTiles, ntl - k0);
    // tile sums: wave w takes tiles w, w + 8, w + 16, w + 24
    for (int kk = wave; kk < kTkTiles; kk += 8) {
      int32_t s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (kk < cnt) {  // wave-uniform
        const int row = min(max(Lt[(long long)(k0 + kk) * kBlock + lane], 0),
                            a.N - 1);
        fx_sum_rows64(kbase, row, lane, s);
      }
      if (lane < 16) {
        float4* dst = reinterpret_cast<float4*>(&ks[kk][8 * lane]);
        dst[0] = make_float4((float)s[0], (float)s[1], (float)s[2], (float)s[3]);
        dst[1] = make_float4((float)s[4], (float)s[5], (float)s[6], (float)s[7]);
      }
    }
    __syncthreads();
    // scores of the wave's 16 blocks against the 32 tiles: two 16 x 16
    // output tiles, 32 k-steps of 4 dims each
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const double bk = (double)ks[16 * c + (lane & 15)][4 * s + (lane >> 4)];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(aq[s], bk, acc, 0, 0, 0);
      }
      // lane l holds the scores of blocks 16 w + 4 r + l / 16 against
      // tile 16 c + l % 16 (the instruction's output layout: item r of
      // lane l is row 4 r + l / 16, column l % 16)
      const int tile = k0 + 16 * c + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * wave + 4 * r + (lane >> 4);
        const int e = chunk * kTkBlocks + j;
        if (e < per_group && tile < ntl) {
          const int h = g * a.G + e % a.G, il = e / a.G;
          const long long bh = (long long)b * a.Hq + h;
          a.scores[bh * per_bh + topk_score_offset(t, il, bps) + tile] =
              (int64_t)acc[r];
        }
      }
    }
    __syncthreads();
  }
}

// One wave per query block: the min(K, ntl) best tiles of L_t by (score
// descending, position ascending), as a bitmask over the positions, and
// their count in n_I. Key of a tile: ((r + 2^49) << 11 | (2047 - position))
// + 1, unique and ordered like (r, -position); 0 marks lanes past the end.
// The K-th largest key T is found bit by bit from the top (at each bit,
// count the keys that agree with the bits found so far and have the bit
// set); the selected tiles are the keys >= T.
__global__ __launch_bounds__(256) void k_topk_select(TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nb = a.N / kBlock;
  if (blk >= (long long)a.B * a.Hq * nb) return;  // wave-uniform
  const long long bh = blk / nb;
  const int I = (int)(blk % nb);
  const int bps = a.S / kBlock;
  const int t = I / bps, ntl = t * bps;
  const int K = min(a.K, ntl);
  uint32_t* mask = a.tmask + blk * kMaskWords;
  if (lane == 0) a.n_I[blk] = K;
  if (K == ntl || K == 0) {  // all or nothing: no ranking needed
#pragma unroll
    for (int i = 0; i < kMaskWords / 64; ++i) {
      const int w = lane + 64 * i;
      const int lo = 32 * w;
      uint32_t bits = 0u;
      if (K > 0 && lo < ntl)
        bits = ntl - lo >= 32 ? 0xffffffffu : ((1u << (ntl - lo)) - 1u);
      mask[w] = bits;
    }
    return;
  }
  const long long per_bh = (long long)bps * bps * a.T * (a.T - 1) / 2;
  const int64_t* sc = a.scores + bh * per_bh +
                      topk_score_offset(t, I - t * bps, bps);
  constexpr int kPer = kMaxTiles / 64;  // positions per lane
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pos = lane + 64 * i;
    key[i] = 0;
    if (pos < ntl)
      key[i] = ((((uint64_t)(sc[pos] + (1ll << 49))) << 11) |
                (uint64_t)(2047 - pos)) + 1;
  }
  uint64_t prefix = 0, msk = 0;
  int want = K;
  for (int bit = 61; bit >= 0; --bit) {
    const uint64_t m = msk | (1ull << bit), cand = prefix | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) c += (key[i] & m) == cand ? 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) c += __shfl_xor(c, o);
    if (c >= want)
      prefix = cand;
    else
      want -= c;
    msk = m;
  }
  // prefix is now the K-th largest key
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint64_t sel = __builtin_amdgcn_ballot_w64(key[i] >= prefix &&
                                                    key[i] != 0);
    // positions 64 i .. 64 i + 63 are words 2 i and 2 i + 1
    if (lane == 0) mask[2 * i] = (uint32_t)sel;
    if (lane == 1) mask[2 * i + 1] = (uint32_t)(sel >> 32);
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int bps = a.S / kBlock;
  const int n_chunk = (a.G * bps + kTkBlocks - 1) / kTkBlocks;
  if (a.T > 1) {
    const long long wgs = (long long)n_chunk * a.B * a.Hkv * (a.T - 1);
    hipLaunchKernelGGL(k_topk_scores, dim3((unsigned)wgs), dim3(512), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nblk = (long long)a.B * a.Hq * (a.N / kBlock);
  hipLaunchKernelGGL(k_topk_select, dim3((unsigned)((nblk + 3) / 4)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t topk_scratch_bytes(int B, int Hq, int S, int T) {
  const size_t bps = (size_t)S / kBlock;
  return (size_t)B * Hq * bps * bps * T * (T - 1) / 2 * sizeof(int64_t);
}

}  // namespace sa
