// Stop points of the early stop, evaluated from pooled means before the
// attention launch.
//
// S2O page, Summary: key/value blocks are visited from the most to the least
// important and a query block stops once the next block's estimated share of
// the attention mass falls below tau. The estimate of a 64 x 64 tile is its
// mean-pooled logit, kappa * qbar_I . kbar_tile, which by linearity is the
// mean of the tile's 4096 logits; the running share compares estimates only
// (the dense local window's estimate, then the visited tiles'). The whole
// stop sequence of a block is therefore a function of three pooled
// quantities: the block's mean query, the mean keys of its segment's 64-key
// blocks and the mean keys of the tiles of L_t. This file computes them and
// scans the sequence, so the attention kernel receives each block's stop
// point n_I and its loop carries no cross-wave decision.
//
//   k_block_qsum : sum of the 64 query rows of every block of pi_Q (fp32);
//   k_stop_scan  : per (b, KV head, segment) and up to 128 query blocks, the
//                  local-window estimate, then the tiles of L_t in visiting
//                  order, 32 at a time: key sums of the tiles (gathered rows,
//                  fp32) in LDS, the mean logits of every block against the
//                  32 tiles as one [128 x 128] x [128 x 32] product on the
//                  matrix cores (v_mfma_f64_16x16x4f64), then per block the
//                  estimates and the share test in float64; stops once every
//                  block has stopped.
//
// Arithmetic (shared with nothing else): a tile's mean logit is
// (qsum . ksum) * kappa / 4096 with both sums in fp32 over bf16 inputs and
// their dot product in float64 (each product of two fp32 values is exact in
// float64; the matrix core sums them in float64). The share E_k / (Acc + E_k) does not depend
// on a common factor of the estimates, so every estimate is taken relative
// to a running reference, the largest mean logit seen so far (the running
// total is rescaled when it rises): exp2 of a non-positive argument in fp32,
// never overflowing and never 0 for the largest term, whatever the scale of
// the logits. The running total and the share test are in float64, the test
// as est < tau * (acc + est).

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kScanBlocks = 128;  // query blocks per scan workgroup
constexpr int kScanThreads = 4 * kScanBlocks;
constexpr int kScanTiles = 32;    // tiles whose key sums sit in LDS at once
constexpr int kSumStride = 132;   // LDS row stride (floats) of the key sums
constexpr int kLogitStride = 33;  // LDS row stride (doubles) of the logits
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Adds the 8 bfloat16 of one 16-byte load to s[0..7].
static __device__ __forceinline__ void add_bf16x8(float (&s)[8], uint4 w) {
  s[0] += bf16_bits_to_f32(w.x & 0xffffu);
  s[1] += bf16_bits_to_f32(w.x >> 16);
  s[2] += bf16_bits_to_f32(w.y & 0xffffu);
  s[3] += bf16_bits_to_f32(w.y >> 16);
  s[4] += bf16_bits_to_f32(w.z & 0xffffu);
  s[5] += bf16_bits_to_f32(w.z >> 16);
  s[6] += bf16_bits_to_f32(w.w & 0xffffu);
  s[7] += bf16_bits_to_f32(w.w >> 16);
}

// Sum of the 64 rows `row_of_lane` names (row r is held by lane r) of a
// [*, 128] bf16 matrix: lane l adds 16-byte chunk l % 16 of rows l / 16,
// l / 16 + 4, ... (ascending), then the four row groups are added across
// lanes (l ^ 16, then l ^ 32). Lanes 0..15 return dims 8 (l % 16) .. + 7;
// every lane of a 16-lane column ends with the same bits.
static __device__ __forceinline__ void sum_rows64(const uint16_t* base,
                                           int row_of_lane, int lane,
                                           float (&s)[8]) {
  const int c = lane & 15, rg = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
  // two batches of 8 loads (fewer registers held), added in row order
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
    for (int j = 0; j < 8; ++j) add_bf16x8(s, w[j]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] += __shfl_xor(s[e], 16);
    s[e] += __shfl_xor(s[e], 32);
  }
}

// Sum over the four lanes of an aligned quad (DPP quad permutations).
static __device__ __forceinline__ int quad_sum_int(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);
  return x;
}

// One wave per query block: qsum[bh][I][:] = sum of the block's 64 rows.
__global__ __launch_bounds__(256) void k_block_qsum(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ pi_q,
    float* __restrict__ qsum, int N, long long n_blocks) {
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= n_blocks) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int nb = N / kBlock;
  const long long bh = blk / nb;
  const int I = (int)(blk % nb);
  const int row = min(max(pi_q[bh * N + (long long)I * kBlock + lane], 0),
                      N - 1);
  float s[8];
  sum_rows64(q + bh * (long long)N * kHeadDim, row, lane, s);
  if (lane < 16) {
    float4* dst = reinterpret_cast<float4*>(qsum + blk * kHeadDim + 8 * lane);
    dst[0] = make_float4(s[0], s[1], s[2], s[3]);
    dst[1] = make_float4(s[4], s[5], s[6], s[7]);
  }
}

// Stop points of up to 128 query blocks of one (b, KV head g, segment t).
// Thread 4 j + dq serves block slot j and dims 32 dq .. + 31 (and rows
// 16 dq .. + 15 of the block for the visible-pair counts).
// Two workgroups per CU (4 waves per SIMD, at most 128 registers): the scan
// waits on its gathers, and the second workgroup's hide them better than
// the registers the matrix-core operands would keep without the bound.
__global__ __launch_bounds__(kScanThreads, 4) void k_stop_scan(StopArgs a) {
  __shared__ __attribute__((aligned(16))) float ksum[kScanTiles][kSumStride];
  // mean logits (log2 units) of the chunk: block slot x tile
  __shared__ double xl[kScanBlocks][kLogitStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid >> 2, dq = tid & 3;
  const int bps = a.S / kBlock;
  const int per_group = a.G * bps;
  const int n_chunk = (per_group + kScanBlocks - 1) / kScanBlocks;
  const int BH = a.B * a.Hkv;
  // segments in descending t: the longest scans start first
  const int p = blockIdx.x;
  const int t = a.T - 1 - p / (n_chunk * BH);
  const int rem = p % (n_chunk * BH);
  const int bg = rem / n_chunk, chunk = rem % n_chunk;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int e = chunk * kScanBlocks + j;
  const bool valid = e < per_group;
  const int h = g * a.G + (valid ? e % a.G : 0);
  const int I = t * bps + (valid ? e / a.G : 0);
  const long long bh = (long long)b * a.Hq + h;
  int32_t* nout = a.n_I + bh * (a.N / kBlock) + I;
  const int ntl = t * bps;  // tiles of L_t

  if (a.fixed >= 0 || t == 0) {  // no estimate decides: a fixed count
    if (valid && dq == 0) *nout = t == 0 ? 0 : min(a.fixed, ntl);
    return;
  }

  // the wave's A operands of the logit product for the whole run: lane l
  // holds block slot 16 w + l % 16, dims 4 s + l / 16 (s = 0..31) of its
  // query sum (0 for slots past the group)
  float aq[32];
  {
    const int ja = 16 * wave + (lane & 15);
    const int ea = chunk * kScanBlocks + ja;
    const bool va = ea < per_group;
    const int ha = g * a.G + (va ? ea % a.G : 0);
    const int Ia = t * bps + (va ? ea / a.G : 0);
    const float* src = a.qsum +
                       (((long long)b * a.Hq + ha) * (a.N / kBlock) + Ia) *
                           kHeadDim + (lane >> 4);
#pragma unroll
    for (int s = 0; s < 32; ++s) aq[s] = va ? src[4 * s] : 0.f;
  }
  const int seg0 = t * a.S;
  const int32_t* pq = a.pi_q + bh * a.N + (long long)I * kBlock + 16 * dq;

  const uint16_t* kbase = a.k + (long long)bg * a.N * kHeadDim;
  const int32_t* Lt = a.L + (long long)bg * a.list_len +
                      (long long)a.S * t * (t - 1) / 2;
  const double c2k = (double)a.c2 / (double)(kBlock * kBlock);

  // key sums of tiles first .. first + 31 of a sequence into LDS; wave w
  // takes tiles w, w + 8, w + 16, w + 24
  auto load_sums = [&](bool local, int first, int count) {
    for (int kk = wave; kk < kScanTiles; kk += 8) {
      if (kk >= count) break;  // wave-uniform
      const int k = first + kk;
      const int row = local ? seg0 + k * kBlock + lane
                            : min(max(Lt[(long long)k * kBlock + lane], 0),
                                  a.N - 1);
      float s[8];
      sum_rows64(kbase, row, lane, s);
      if (lane < 16) {
        float4* dst = reinterpret_cast<float4*>(&ksum[kk][8 * lane]);
        dst[0] = make_float4(s[0], s[1], s[2], s[3]);
        dst[1] = make_float4(s[4], s[5], s[6], s[7]);
      }
    }
  };
  // the mean logits of the 128 block slots against the 32 tiles in LDS, in
  // log2 units: (qsum . ksum) kappa log2(e) / 4096, the products exact in
  // float64 and summed in float64 (no error that grows with the size of the
  // logits). Wave w: slots 16 w .. + 15, two 16 x 16 output tiles, 32
  // k-steps of 4 dims; B operands: lane l holds tile 16 c + l % 16, dims
  // 4 s + l / 16. Item r of lane l is slot 16 w + 4 r + l / 16, tile
  // 16 c + l % 16 (the instruction's output layout). Every wave runs it.
  auto chunk_logits = [&]() {
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
    const float* b0 = &ksum[lane & 15][lane >> 4];
    const float* b1 = &ksum[16 + (lane & 15)][lane >> 4];
#pragma unroll 8
    for (int s = 0; s < 32; ++s) {
      const double av = (double)aq[s];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)b0[4 * s], acc0,
                                                  0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)b1[4 * s], acc1,
                                                  0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xl[16 * wave + 4 * r + (lane >> 4)][lane & 15] = acc0[r] * c2k;
      xl[16 * wave + 4 * r + (lane >> 4)][16 + (lane & 15)] = acc1[r] * c2k;
    }
  };
  auto tile_x = [&](int kk) { return xl[j][kk]; };
  // estimates relative to the running reference ref (the largest mean
  // logit so far): exp2(x - ref) after raising ref to x if needed, with the
  // running total acc (relative to ref as well) rescaled then
  double ref = -INFINITY;
  auto rel_exp = [&](double x, double& acc) {
    if (x > ref) {
      acc *= (double)__builtin_amdgcn_exp2f((float)(ref - x));  // 0 at first
      ref = x;
    }
    return (double)__builtin_amdgcn_exp2f((float)(x - ref));
  };

  // dense local window: E_diag = sum over the segment's 64-key blocks c, in
  // ascending order, of (visible pairs / 64) * exp(mean logit)
  double acc = 0.0;
  for (int c0 = 0; c0 < bps; c0 += kScanTiles) {
    const int cnt = min(kScanTiles, bps - c0);
    __syncthreads();
    load_sums(true, c0, cnt);
    __syncthreads();
    chunk_logits();
    __syncthreads();
    if (valid) {
      // this thread's 16 rows (offsets from the segment start)
      int rofs[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        rofs[i] = min(max(pq[i], 0), a.N - 1) - seg0;
      for (int kk = 0; kk < cnt; ++kk) {
        const int j0 = (c0 + kk) * kBlock;
        int nv = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) nv += min(max(rofs[i] - j0 + 1, 0), kBlock);
        nv = quad_sum_int(nv);
        const double x = tile_x(kk);
        if (nv > 0) {
          const double ex = rel_exp(x, acc);
          acc += ((double)nv / kBlock) * ex;
        }
      }
    }
  }

  // tiles of L_t in visiting order: share est / (acc + est) < tau stops
  bool active = valid;
  int n = ntl;
  for (int k0 = 0; k0 < ntl; k0 += kScanTiles) {
    if (!__syncthreads_or(active)) break;
    const int cnt = min(kScanTiles, ntl - k0);
    load_sums(false, k0, cnt);
    __syncthreads();
    chunk_logits();
    __syncthreads();
    if (active) {
      for (int kk = 0; kk < cnt; ++kk) {
        const double est = kBlock * rel_exp(tile_x(kk), acc);
        if (est < a.tau * (acc + est)) {
          n = k0 + kk;
          active = false;
          break;
        }
        acc += est;
      }
    }
  }
  if (valid && dq == 0) *nout = n;
}

// Order of the query blocks of one (b, KV head, segment) group for the
// sparse attention pass: stop point descending, block index ascending on
// ties. A workgroup takes 4 consecutive blocks of this order, so its blocks
// stop at nearly the same step (a workgroup runs to its largest stop
// point). One workgroup per group; rank by counting, P <= kOrderMax.
__global__ __launch_bounds__(256) void k_block_order(const int32_t* __restrict__ n_I,
                                                     int32_t* __restrict__ order,
                                                     int Hq, int Hkv, int N,
                                                     int S, int T, int G) {
  __shared__ int nv[kOrderMax];
  const int grp = blockIdx.x;  // bg * T + t
  const int bg = grp / T, t = grp % T, b = bg / Hkv, g = bg % Hkv;
  const int bps = S / kBlock, P = G * bps;
  for (int e = threadIdx.x; e < P; e += 256) {
    const int h = g * G + e % G, I = t * bps + e / G;
    nv[e] = n_I[((long long)b * Hq + h) * (N / kBlock) + I];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < P; e += 256) {
    const int v = nv[e];
    int r = 0;
    for (int j = 0; j < P; ++j) {
      const int w = nv[j];
      r += (w > v || (w == v && j < e)) ? 1 : 0;
    }
    order[(long long)grp * P + r] = e;
  }
}

hipError_t launch_block_order(const PlanDims& d, const int32_t* n_I,
                              int32_t* order, hipStream_t s) {
  hipLaunchKernelGGL(k_block_order, dim3(d.B * d.Hkv * d.T), dim3(256), 0, s,
                     n_I, order, d.Hq, d.Hkv, d.N, d.S, d.T, d.G);
  return hipGetLastError();
}

hipError_t launch_block_qsum(const PlanDims& d, const uint16_t* q,
                             const int32_t* pi_q, float* qsum, hipStream_t s) {
  const long long nblk = (long long)d.B * d.Hq * (d.N / kBlock);
  hipLaunchKernelGGL(k_block_qsum, dim3((unsigned)((nblk + 3) / 4)),
                     dim3(256), 0, s, q, pi_q, qsum, d.N, nblk);
  return hipGetLastError();
}

hipError_t launch_stop_scan(const StopArgs& a, hipStream_t s) {
  const int bps = a.S / kBlock;
  const int n_chunk = (a.G * bps + kScanBlocks - 1) / kScanBlocks;
  const long long wgs = (long long)n_chunk * a.B * a.Hkv * a.T;
  hipLaunchKernelGGL(k_stop_scan, dim3((unsigned)wgs), dim3(kScanThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace sa
