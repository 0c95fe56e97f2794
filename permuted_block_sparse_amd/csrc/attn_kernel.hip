// Gather attention with the early stop (S2O page, Summary): the kernel
// fetches the indexed tokens into on-chip memory (LDS), processes key/value
// blocks from most to least important with an online softmax (FlashAttention
// tiling) and stops a query block once the next block's estimated share of
// the attention mass falls below tau. Outputs go back to their original rows
// (no tensor is moved).
//
// Work decomposition (gfx950, wave64): one workgroup = 4 waves = 4 query
// blocks of 64 rows that share the same KV head g and segment t, hence the
// same key tiles (dense local window = segment t's keys; sparse tiles =
// L_t). Each wave owns one whole query block, so the stop test of a block
// is wave-local. K and V tiles are gathered into LDS once per workgroup and
// read by all 4 waves.
//
// Per wave and 64-key tile:
//   S^T = K Q^T   : 2 x 2 v_mfma_f32_32x32x16_bf16 blocks over d = 128
//                   (Q^T held in registers as B operands for the whole run);
//   mean of S     : the mean-pooled logit of the tile (the block estimate);
//   online softmax: per-lane rows (lane = query), fp32, exp2 domain;
//   O^T += V^T P^T: V^T A operands from LDS via ds_read_tr16_b64 transposed
//                   reads, P^T B operands straight from the S registers.

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kLdsStride = 136;  // bf16 per LDS row: 256 B + 16 B pad

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum with the lane 32 apart (the other half of the same query row).
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
  x = sum_xor32(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                       __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Cooperative gather of 64 K rows and 64 V rows into LDS. Rows are the keys
// `idx[0..63]` (sparse tile) or j0 .. j0 + 63 (local block). 16 lanes move
// one 256-byte row with 16-byte loads.
__device__ __forceinline__ void load_tile(uint16_t* Ks, uint16_t* Vs,
                                          const uint16_t* kbase,
                                          const uint16_t* vbase,
                                          const int32_t* idx, int j0,
                                          int nkeys) {
  const int c = threadIdx.x & 15, r = threadIdx.x >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = r + 16 * p;
    int key = idx != nullptr ? idx[row] : j0 + row;
    key = min(max(key, 0), nkeys - 1);  // memory-safe for any index array
    const uint4 kk =
        *reinterpret_cast<const uint4*>(kbase + (size_t)key * kHeadDim + 8 * c);
    const uint4 vv =
        *reinterpret_cast<const uint4*>(vbase + (size_t)key * kHeadDim + 8 * c);
    *reinterpret_cast<uint4*>(Ks + row * kLdsStride + 8 * c) = kk;
    *reinterpret_cast<uint4*>(Vs + row * kLdsStride + 8 * c) = vv;
  }
}

// S^T[kb][qb]: keys kb*32 + 8(r/4) + 4 lh + r%4, queries qb*32 + lq.
__device__ __forceinline__ void qk_tile(const uint16_t* Ks,
                                        const bf16x8 (&qr)[2][8],
                                        f32x16 (&sacc)[2][2], int lq, int lh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
          Ks + (kb * 32 + lq) * kLdsStride + 16 * s + 8 * lh);
      sacc[kb][0] = mfma32(ka, qr[0][s], sacc[kb][0]);
      sacc[kb][1] = mfma32(ka, qr[1][s], sacc[kb][1]);
    }
  }
}

__device__ __forceinline__ float tile_sum(const f32x16 (&sacc)[2][2]) {
  float s = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += sacc[kb][qb][r];
  return wave_sum(s);
}

// Online softmax update of the two query rows of this lane, then
// O^T += V^T P^T. m is kept in the exp2 domain (m = max logit * c2).
__device__ __forceinline__ void softmax_pv(const uint16_t* Vs,
                                           f32x16 (&sacc)[2][2],
                                           f32x16 (&oacc)[4][2], float (&m)[2],
                                           float (&l)[2], float c2, int lane) {
  const int lh = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
    mx = max_xor32(mx);
    const float mnew = fmaxf(m[qb], mx * c2);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m[qb] - muse);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[kb][qb][r] * c2 - muse);
        sacc[kb][qb][r] = p;
        rs += p;
      }
    rs = sum_xor32(rs);
    l[qb] = l[qb] * alpha + rs;
    m[qb] = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db][qb] *= alpha;
  }
  // tr16 source address of this lane: key row 4 lh + i/4 (+8), column
  // 16 ((lane >> 4) & 1) + 4 (i % 4) within the 32-column block db.
  const int i16 = lane & 15;
  const int col = 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
  const int rowo = 4 * lh + (i16 >> 2);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kb = s >> 1, half = s & 1;
    bf16x8 pb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[qb][e] = (__bf16)sacc[kb][qb][8 * half + e];
    const uint16_t* vrow = Vs + (32 * kb + 16 * half + rowo) * kLdsStride + col;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const s16x4 lo = lds_read_tr16(vrow + 32 * db);
      const s16x4 hi = lds_read_tr16(vrow + 8 * kLdsStride + 32 * db);
      const s16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 va = __builtin_bit_cast(bf16x8, cat);
      oacc[db][0] = mfma32(va, pb[0], oacc[db][0]);
      oacc[db][1] = mfma32(va, pb[1], oacc[db][1]);
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_attn_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kBlock * kLdsStride];
  __shared__ int wave_maxrow[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lh = lane >> 5;

  // ---- which (b, g, t) group and which 4 query blocks.
  // Groups are ranked by descending t (longest work first). Consecutive
  // workgroup ids are dispatched round-robin over the 8 XCDs; group q runs on
  // XCD q % 8 so that all workgroups of one group share that XCD's L2.
  const int p = blockIdx.x;
  int grp, chunk;
  if ((a.n_groups & 7) == 0) {
    const int x = p & 7, slot = p >> 3;
    grp = x + 8 * (slot / a.wg_per_group);
    chunk = slot % a.wg_per_group;
  } else {
    grp = p / a.wg_per_group;
    chunk = p % a.wg_per_group;
  }
  const int BH = a.B * a.Hkv;
  const int t = a.T - 1 - grp / BH;
  const int bg = grp % BH, b = bg / a.Hkv, g = bg % a.Hkv;
  const int bps = a.S / kBlock;  // query blocks per segment and head
  const int e = chunk * 4 + wave;
  const bool valid = e < a.G * bps;
  const int h = g * a.G + (valid ? e % a.G : 0);
  const int I = t * bps + (valid ? e / a.G : 0);

  const size_t bh = (size_t)b * a.Hq + h;
  const int32_t* pq = a.pi_q + bh * a.N + (size_t)I * kBlock;
  const int iq0 = min(max(pq[lq], 0), a.N - 1);
  const int iq1 = min(max(pq[32 + lq], 0), a.N - 1);
  const uint16_t* qh = a.q + bh * a.N * kHeadDim;
  bf16x8 qr[2][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qr[0][s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)iq0 * kHeadDim +
                                                16 * s + 8 * lh);
    qr[1][s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)iq1 * kHeadDim +
                                                16 * s + 8 * lh);
  }
  const uint16_t* kbase = a.k + (size_t)bg * a.N * kHeadDim;
  const uint16_t* vbase = a.v + (size_t)bg * a.N * kHeadDim;

  f32x16 oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db][0] = oacc[db][1] = f32x16{};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x16 sacc[2][2];
  double acc = 0.0;  // running estimated mass (dense window + visited tiles)

  // ---- dense local window: keys of segment t, causal mask j <= row.
  const int seg0 = t * a.S;
  const int myrow = wave_max_int(max(iq0, iq1));
  if (lane == 0) wave_maxrow[wave] = valid ? myrow : -1;
  __syncthreads();
  const int wgmax = max(max(wave_maxrow[0], wave_maxrow[1]),
                        max(wave_maxrow[2], wave_maxrow[3]));
  const int ndiag = min(max((wgmax - seg0) / kBlock + 1, 1), bps);
  for (int c = 0; c < ndiag; ++c) {
    const int j0 = seg0 + c * kBlock;
    const int nv_lane =
        lh == 0 ? min(max(iq0 - j0 + 1, 0), kBlock) +
                      min(max(iq1 - j0 + 1, 0), kBlock)
                : 0;
    const int nvis = wave_sum_int(nv_lane);
    load_tile(Ks, Vs, kbase, vbase, nullptr, j0, a.N);
    __syncthreads();
    if (valid && nvis > 0) {
      qk_tile(Ks, qr, sacc, lq, lh);
      const float ssum = tile_sum(sacc);
      acc += ((double)nvis / kBlock) *
             exp((double)ssum * (a.kappa / (kBlock * kBlock)));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jk = j0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (jk > iq0) sacc[kb][0][r] = -INFINITY;
          if (jk > iq1) sacc[kb][1][r] = -INFINITY;
        }
      softmax_pv(Vs, sacc, oacc, m, l, a.c2, lane);
    }
    __syncthreads();
  }

  // ---- sparse tiles of L_t, most to least important, until the stop.
  int n_visit = 0;
  if (t > 0) {
    const int ntiles = t * bps;
    const int32_t* Lt =
        a.L + (size_t)bg * a.list_len + (size_t)a.S * t * (t - 1) / 2;
    bool active = valid;
    n_visit = ntiles;
    for (int kt = 0; kt < ntiles; ++kt) {
      load_tile(Ks, Vs, kbase, vbase, Lt + (size_t)kt * kBlock, 0, a.N);
      __syncthreads();
      if (active) {
        qk_tile(Ks, qr, sacc, lq, lh);
        const float ssum = tile_sum(sacc);
        const double est =
            kBlock * exp((double)ssum * (a.kappa / (kBlock * kBlock)));
        if (est / (acc + est) < a.tau) {
          active = false;
          n_visit = kt;
        } else {
          acc += est;
          softmax_pv(Vs, sacc, oacc, m, l, a.c2, lane);
        }
      }
      if (!__syncthreads_or(active)) break;
    }
  }

  // ---- epilogue: normalise, round to bf16, scatter to the original rows.
  if (!valid) return;
  const float ln2 = 0.69314718055994530942f;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb ? iq1 : iq0;
    const float inv = 1.f / l[qb];
    uint16_t* orow = a.o + (bh * a.N + row) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * lh;
        __bf16 v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(oacc[db][qb][4 * g4 + j] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = __builtin_bit_cast(uint2, v4);
      }
    if (a.lse != nullptr && lh == 0)
      a.lse[bh * a.N + row] = (m[qb] + log2f(l[qb])) * ln2;
  }
  if (lane == 0) a.n_out[bh * (a.N / kBlock) + I] = n_visit;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int total = a.n_groups * a.wg_per_group;
  hipLaunchKernelGGL(k_attn_fwd, dim3(total), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
