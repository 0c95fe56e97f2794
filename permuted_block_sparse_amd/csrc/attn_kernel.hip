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
// Pipeline: the local blocks and then the sparse tiles form one sequence of
// steps. While step s is computed from LDS buffer s % 2, the gather of step
// s + 1 streams into the other buffer with direct global->LDS loads (no
// registers), and the tile indices of step s + 2 are fetched; one barrier
// per step.
//
// Per wave and 64-key tile:
//   S^T = K Q^T   : 2 x 2 v_mfma_f32_32x32x16_bf16 blocks over d = 128
//                   (Q^T held in registers as B operands for the whole run);
//   mean of S     : the mean-pooled logit of the tile (the block estimate);
//   online softmax: per-lane rows (lane = query), fp32, exp2 domain; the
//                   running max is only raised when a row's max exceeds it
//                   by more than 2^8 (exact: o = acc / l for any reference);
//   O^T += V^T P^T: V^T A operands from LDS via ds_read_tr16_b64 transposed
//                   reads, P^T B operands straight from the S registers.
//
// LDS layouts are "read-native": each tile is stored in exactly the order in
// which the MFMA operand reads consume it, so every LDS read instruction of
// a wave touches one contiguous 1 KB (K, ds_read_b128) or 512 B (V,
// ds_read_tr16_b64) block -- free of bank conflicts, and every read address
// is a per-lane base plus an immediate. The gather side picks, per lane,
// the global 16-byte chunk that belongs at its LDS slot.
//   K tile: block (kb, s) of 1 KB at (8 kb + s) KB; lane l's 16 bytes hold
//           K[row 32 kb + l % 32][elements 16 s + 8 (l / 32) .. + 7].
//   V tile: block id = ((2 kb + half) 4 + db) 2 + hi of 512 B at 512 id;
//           lane l's 8 bytes hold the 4 elements the transposed read of
//           lane l takes: V[row 32 kb + 16 half + 4 (l / 32) + (l % 16) / 4
//           + 8 hi][col 32 db + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3].

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kTileBytes = kBlock * kHeadDim * 2;  // 16 KB: one K or V tile
constexpr float kRescaleSlack = 8.0f;              // log2 units

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

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Rows of the K and V tiles whose chunks lane `lane` of wave `wave` moves
// (one row each per step; see the layouts above).
__device__ __forceinline__ int gather_row_k(int wave, int lane) {
  return 32 * (wave >> 1) + (lane & 31);
}
__device__ __forceinline__ int gather_row_v(int wave, int lane) {
  return 16 * wave + 4 * ((lane >> 4) & 1) + ((lane & 7) >> 1) +
         8 * (lane >> 5);
}

// Issue the gather of one K tile and one V tile into LDS (asynchronous,
// completion tracked by the vector memory counter): wave w writes K blocks
// 4 w .. 4 w + 3 and V blocks 8 w .. 8 w + 7, 1 KB per instruction.
__device__ __forceinline__ void issue_gather(char* kdst, char* vdst,
                                             const uint16_t* kbase,
                                             const uint16_t* vbase, int key_k,
                                             int key_v, int wave, int lane) {
  const uint16_t* krow = kbase + (size_t)key_k * kHeadDim + 8 * (lane >> 5);
  const uint16_t* vrow = vbase + (size_t)key_v * kHeadDim +
                         8 * (2 * ((lane >> 3) & 1) + (lane & 1));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * (wave & 1) + j;  // K block (wave / 2, s)
    __builtin_amdgcn_global_load_lds(
        krow + 16 * s, (lds_void*)(kdst + (8 * (wave >> 1) + s) * 1024), 16,
        0, 0);
    // V write block 4 w + j holds tr16 blocks 8 w + 2 j (+1), db = j
    __builtin_amdgcn_global_load_lds(
        vrow + 32 * j, (lds_void*)(vdst + (4 * wave + j) * 1024), 16, 0, 0);
  }
}

// S^T[kb][qb]: keys kb*32 + 8(r/4) + 4 lh + r%4, queries qb*32 + lq.
// Q^T operands come from the wave's own LDS copy of its query block, laid
// out like the K tile: block (qb, s) of 1 KB, lane l's 16 bytes =
// Q[row qb*32 + l % 32][elements 16 s + 8 (l / 32) .. + 7].
__device__ __forceinline__ void qk_tile(const char* Kt, const char* Qw,
                                        f32x16 (&sacc)[2][2], int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8 q0 =
        *reinterpret_cast<const bf16x8*>(Qw + s * 1024 + 16 * lane);
    const bf16x8 q1 =
        *reinterpret_cast<const bf16x8*>(Qw + (8 + s) * 1024 + 16 * lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
          Kt + (8 * kb + s) * 1024 + 16 * lane);
      sacc[kb][0] = mfma32(ka, q0, sacc[kb][0]);
      sacc[kb][1] = mfma32(ka, q1, sacc[kb][1]);
    }
  }
}

__device__ __forceinline__ float tile_sum(const f32x16 (&sacc)[2][2]) {
  // pairwise tree over the 64 values of this lane
  f32x16 t = (sacc[0][0] + sacc[0][1]) + (sacc[1][0] + sacc[1][1]);
  float s8[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) s8[r] = t[r] + t[r + 8];
  const float s = ((s8[0] + s8[4]) + (s8[1] + s8[5])) +
                  ((s8[2] + s8[6]) + (s8[3] + s8[7]));
  return wave_sum(s);
}

// Online softmax update of the two query rows of this lane, then
// O^T += V^T P^T. m is kept in the exp2 domain (m = reference logit * c2).
__device__ __forceinline__ void softmax_pv(const char* Vt,
                                           f32x16 (&sacc)[2][2],
                                           f32x16 (&oacc)[4][2], float (&m)[2],
                                           float (&l)[2], float c2, int lane) {
  const int lh = lane >> 5;
  float mx[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float v = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[kb][qb][r]);
    mx[qb] = max_xor32(v) * c2;
  }
  // raise the reference only when some row's max exceeds it by > 2^8
  const bool raise = (mx[0] > m[0] + kRescaleSlack) ||
                     (mx[1] > m[1] + kRescaleSlack);
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mnew = fmaxf(m[qb], mx[qb]);
      // 0 when m was -inf; 1 when unchanged (also when both are -inf)
      const float alpha = m[qb] == mnew ? 1.f : exp2f(m[qb] - mnew);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db][qb] *= alpha;
      m[qb] = mnew;
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // m is finite here for every row that has seen a visible key; a row
    // with none yet has only masked (-inf) logits, whose p is 0 for any
    // finite reference
    const float muse = m[qb] == -INFINITY ? 0.f : m[qb];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][qb][r] * c2 - muse);
        sacc[kb][qb][r] = p;
        rs += p;
      }
    l[qb] += sum_xor32(rs);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kb = s >> 1, half = s & 1;
    bf16x8 pb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[qb][e] = (__bf16)sacc[kb][qb][8 * half + e];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int id = ((2 * kb + half) * 4 + db) * 2;
      const s16x4 lo = lds_read_tr16(Vt + id * 512 + 8 * lane);
      const s16x4 hi = lds_read_tr16(Vt + (id + 1) * 512 + 8 * lane);
      const s16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 va = __builtin_bit_cast(bf16x8, cat);
      oacc[db][0] = mfma32(va, pb[0], oacc[db][0]);
      oacc[db][1] = mfma32(va, pb[1], oacc[db][1]);
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_attn_fwd(AttnArgs a) {
  // K/V double buffer (4 x 16 KB) + one 16 KB query block per wave
  extern __shared__ __attribute__((aligned(1024))) char smem[];
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
  // the wave's query block -> its own 16 KB of LDS (B-operand order)
  char* Qw = smem + 4 * kTileBytes + wave * kTileBytes;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    __builtin_amdgcn_global_load_lds(
        qh + (size_t)iq0 * kHeadDim + 16 * s + 8 * lh,
        (lds_void*)(Qw + s * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        qh + (size_t)iq1 * kHeadDim + 16 * s + 8 * lh,
        (lds_void*)(Qw + (8 + s) * 1024), 16, 0, 0);
  }
  const uint16_t* kbase = a.k + (size_t)bg * a.N * kHeadDim;
  const uint16_t* vbase = a.v + (size_t)bg * a.N * kHeadDim;

  f32x16 oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db][0] = oacc[db][1] = f32x16{};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x16 sacc[2][2];
  double acc = 0.0;  // running estimated mass (dense window + visited tiles)

  // ---- the step sequence: ndiag local blocks, then the tiles of L_t.
  const int seg0 = t * a.S;
  const int myrow = wave_max_int(max(iq0, iq1));
  if (lane == 0) wave_maxrow[wave] = valid ? myrow : -1;
  __syncthreads();
  const int wgmax = max(max(wave_maxrow[0], wave_maxrow[1]),
                        max(wave_maxrow[2], wave_maxrow[3]));
  const int ndiag = min(max((wgmax - seg0) / kBlock + 1, 1), bps);
  const int ntiles = t * bps;
  const int nsteps = ndiag + ntiles;
  const int32_t* Lt =
      a.L + (size_t)bg * a.list_len + (size_t)a.S * t * (t - 1) / 2;

  // key rows this lane gathers for step s
  const int rk = gather_row_k(wave, lane), rv = gather_row_v(wave, lane);
  auto step_key = [&](int s, int row) {
    const int kk = s < ndiag ? seg0 + s * kBlock + row
                             : Lt[(size_t)(s - ndiag) * kBlock + row];
    return min(max(kk, 0), a.N - 1);  // memory-safe for any index array
  };

  int nk_k = 0, nk_v = 0;  // keys of the next step to issue
  issue_gather(smem, smem + kTileBytes, kbase, vbase, step_key(0, rk),
               step_key(0, rv), wave, lane);
  if (nsteps > 1) {
    nk_k = step_key(1, rk);
    nk_v = step_key(1, rv);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  bool active = valid;
  int n_visit = t > 0 ? ntiles : 0;
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const char* Kt = smem + cur * 2 * kTileBytes;
    const char* Vt = Kt + kTileBytes;
    if (s + 1 < nsteps) {
      char* nk = smem + (cur ^ 1) * 2 * kTileBytes;
      issue_gather(nk, nk + kTileBytes, kbase, vbase, nk_k, nk_v, wave,
                   lane);
      if (s + 2 < nsteps) {
        nk_k = step_key(s + 2, rk);
        nk_v = step_key(s + 2, rv);
      }
    }
    // local block (s < ndiag): exact causal attention, mass estimate from
    // the mean logit of the whole 64 x 64 block weighted by its visible
    // pairs; sparse tile: estimate, stop test, then attention.
    const bool local = s < ndiag;
    const int j0 = seg0 + s * kBlock;
    const int nv_lane = (local && lh == 0)
                            ? min(max(iq0 - j0 + 1, 0), kBlock) +
                                  min(max(iq1 - j0 + 1, 0), kBlock)
                            : 0;
    const int nvis = local ? wave_sum_int(nv_lane) : 0;
    const bool work = local ? (valid && nvis > 0) : active;
    if (work) {
      qk_tile(Kt, Qw, sacc, lane);
      const float ssum = tile_sum(sacc);
      const double ex = exp((double)ssum * (a.kappa / (kBlock * kBlock)));
      bool take = true;
      if (local) {
        acc += ((double)nvis / kBlock) * ex;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jk = j0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (jk > iq0) sacc[kb][0][r] = -INFINITY;
            if (jk > iq1) sacc[kb][1][r] = -INFINITY;
          }
      } else {
        const double est = kBlock * ex;
        if (est / (acc + est) < a.tau) {
          active = false;
          n_visit = s - ndiag;
          take = false;
        } else {
          acc += est;
        }
      }
      if (take) softmax_pv(Vt, sacc, oacc, m, l, a.c2, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this step's gather and index loads
    if (!__syncthreads_or(active)) break;
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
        for (int j = 0; j < 4; ++j)
          v4[j] = (__bf16)(oacc[db][qb][4 * g4 + j] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = __builtin_bit_cast(uint2, v4);
      }
    if (a.lse != nullptr && lh == 0)
      a.lse[bh * a.N + row] = (m[qb] + log2f(l[qb])) * ln2;
  }
  if (lane == 0) a.n_out[bh * (a.N / kBlock) + I] = n_visit;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int total = a.n_groups * a.wg_per_group;
  constexpr int kLds = 8 * kTileBytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(k_attn_fwd),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_attn_fwd, dim3(total), dim3(256), kLds, s, a);
  return hipGetLastError();
}

}  // namespace sa
