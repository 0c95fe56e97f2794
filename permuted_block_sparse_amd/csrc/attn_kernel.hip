// Gather attention with the early stop (S2O page, Summary): the kernel
// fetches the indexed tokens into on-chip memory (LDS), processes key/value
// blocks from most to least important with an online softmax (FlashAttention
// tiling) and stops each query block at its stop point n_I, the first tile
// whose estimated share of the attention mass falls below tau. The stop
// points depend only on pooled means and are scanned before this launch;
// the loop itself carries no decision. Outputs go back to their original
// rows (no tensor is moved).
//
// Two passes of one kernel per prefill. The local pass computes each query
// block's dense local window in the rows' own order: block i of segment t
// (rows t S + 64 i ..) against key blocks 0 .. i of the segment, only the
// last one masked. It writes the normalised result to O (bf16), its
// residual below that bf16 value to a scratch array (bf16; the two carry
// about 16 significant bits of the fp32 result; only for half-rows with a
// value of magnitude >= 1, where the rounding would matter) and the
// log2-sum-exp of each row. The sparse pass takes the blocks of pi_Q: each row resumes from
// that state (reference = the local log2-sum-exp, l = 1, accumulator = the
// local output, the bf16 value plus its residual) and continues over the
// first n_I tiles of L_t, then overwrites its row of O, so the output is
// rounded to bf16 once. The softmax does not depend on the order in which
// a row's keys are visited. A block
// of pi_Q holds rows from all over its segment, so in that order its local
// window would need every key block of the segment with about half of the
// pairs masked; in the rows' own order it needs about half as many tiles.
//
// Work decomposition (gfx950, wave64, 2 waves per SIMD): one workgroup = 8
// waves = 4 query blocks of 64 rows that share the same KV head g and
// segment t, hence the same key tiles (local pass: segment t's keys; sparse
// pass: L_t). Wave w holds rows 32 (w / 4) .. + 31 of query block w % 4;
// both halves of a block sit on the same SIMD. K and V tiles are gathered
// into LDS once per workgroup and read by all 8 waves; the workgroup runs to
// the largest step count of its blocks, and a wave whose block is done only
// helps with the gathers. Where the shape allows, the local pass gives each
// workgroup two blocks of the same heads one after the other, blocks i and
// S / 64 - 1 - i of a segment (S / 64 + 1 steps for every workgroup, half
// as many workgroups and their fixed costs).
//
// Pipeline: each wave overlaps its matrix and vector work within a step.
// LDS holds a ring of four K tile buffers and a ring of four V tile buffers
// (tile j in slot j % 4), each wave two sets of logit registers. Step s:
// the reference of tile s (see the online softmax below); the QK MFMAs of
// tile s + 1 interleaved with the exponentials of tile s; the PV MFMAs of
// tile s; the K rows of tile s + 3 and the V rows of tile s + 2 (loaded
// into registers during step s - 1) into the slots of tiles s - 1 and
// s - 2; the loads of the K rows of tile s + 4, the V rows of tile s + 3
// and the indices of tile s + 5. One barrier per pair of steps (s even,
// s + 1): the pair reads K slots s + 1, s + 2 and V slots s, s + 1, and
// writes K slots s + 3, s + 4 and V slots s + 2, s + 3, the four other
// slots of each ring, so the waves of a workgroup may be a step apart
// between barriers. A wave whose block is done (or that holds no rows)
// runs the same instructions as a no-op, so no branch splits the MFMA and
// VALU work.
//
// Exact per-block max mode (the BSFA page's test, instead of the stop): every
// tile of L_t is scored and attended iff the largest logit of the 64 x 64
// tile reaches the threshold. Each half of a block posts its maximum of
// tile s + 1 to LDS right after that tile's QK (one slot per step parity);
// after the barrier both halves take max(own, other) of the same two
// values, so they decide on the same bits without waiting for each other.
//
// Per wave and 64-key tile:
//   S^T = K Q^T   : 2 v_mfma_f32_32x32x16_bf16 blocks over d = 128, Q^T
//                   operands held in registers for the whole run;
//   online softmax: one query row per lane pair (lane, lane ^ 32), fp32,
//                   exp2 domain; o = acc / l holds for any reference, so
//                   the reference is raised only when p values could pass
//                   2^8. The local pass takes the row maximum of every
//                   tile (rescaling lazily). In the sparse pass, rows that
//                   are provably bounded (the logit bound |q| max |k| kappa
//                   log2(e) within 120 of the local log2-sum-exp, so no p
//                   can overflow) skip the per-tile row maximum and test the
//                   lane's tile sum instead (a sum above 2^8 divides the row
//                   by its largest p); workgroups with other rows take the
//                   row maximum of every tile (a further launch);
//   O^T += V^T P^T: fp16 products (P rounded to fp16, 2^-11 relative, and
//                   V read from an fp16 copy, exact for bf16 values of
//                   magnitude in [2^-14, 65504]); V^T A operands via
//                   ds_read_tr16_b64 transposed reads, P^T B operands
//                   straight from the S registers.
//
// LDS layouts follow the MFMA operand reads: each read instruction of a wave
// touches one 1 KB (K, ds_read_b128) or 512 B (V, ds_read_tr16_b64) block,
// with the lanes' 16-byte slots permuted by an XOR swizzle. The gather is by
// whole rows: lane L of wave w moves key row 8 w + L / 8 (its K and its V
// row), 16-byte chunks L % 8 and 8 + L % 8, so each global load instruction
// covers 8 full 128-byte lines. The swizzle makes both the stores of these
// chunks and the operand reads free of bank conflicts (64 banks of 4 bytes,
// 16 lanes of 16 bytes per cycle; also with 32 banks, 8 lanes per cycle).
//   K tile: block (kb, s) of 1 KB at (8 kb + s) KB; lane l's 16 bytes hold
//           K[row 32 kb + l % 32][elements 16 s + 8 (l / 32) .. + 7], at
//           slot l ^ (2 (s % 4) + l / 32) ^ 8 (l % 2).
//   V tile: block id = ((2 kb + half) 4 + db) 2 + hi of 512 B at 512 id;
//           lane l's 8 bytes hold the 4 elements the transposed read of
//           lane l takes: V[row 32 kb + 16 half + 4 (l / 32) + (l % 16) / 4
//           + 8 hi][col 32 db + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3], in
//           half l % 2 of 16-byte slot
//           (l / 2) ^ 2 ((l / 16) % 2) ^ 4 (db % 2).

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

constexpr int kTileBytes = kBlock * kHeadDim * 2;  // 16 KB: one K or V tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;               // log2 units
// A lane's sum of one tile's 32 p values above this means some p may exceed
// 2^kRescaleSlack (every p > 2^8 lifts the sum above it): rescale.
constexpr float kRescaleSum = 256.0f;
// Rows whose logits provably stay below reference + kSafeSpan (log2 units)
// skip the per-tile row maximum: no p can overflow fp32 before the rescale.
constexpr float kSafeSpan = 120.0f;
// The local pass hands each half-row to the sparse pass as bf16 values plus
// bf16 residuals; the residuals are stored and read only when one of the 64
// bf16 values reaches this magnitude.
constexpr float kResidualFrom = 1.0f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Cross-lane exchanges without LDS round trips: DPP within rows of 16,
// permlane swaps across 16 and 32.
__device__ __forceinline__ int dpp_xor1(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad [1,0,3,2]
}
__device__ __forceinline__ int dpp_xor2(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad [2,3,0,1]
}
__device__ __forceinline__ int dpp_half_mirror(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // i <-> 7 - i
}
__device__ __forceinline__ int dpp_mirror(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);  // i <-> 15 - i
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

// Wave-wide maximum, made uniform through lane 0.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(dpp_xor1(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_xor2(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_half_mirror(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_mirror(__float_as_int(x))));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  x = max_xor32(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                       __builtin_bit_cast(int, x)));
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

// The tile row whose K and V chunks lane `lane` of wave `wave` moves.
__device__ __forceinline__ int gather_row(int wave, int lane) {
  return 8 * wave + (lane >> 3);
}

// LDS byte offsets of the two K and two V chunks one lane stores (the second
// of each pair is the first plus 4 KB for K, plus 2 KB for V).
struct StoreAddr {
  int k, v;
};
__device__ __forceinline__ StoreAddr store_addr(int row, int lane) {
  const int c = lane & 7;  // 16-byte chunk of the row's first half
  StoreAddr a;
  {
    const int kb = row >> 5, s = c >> 1, b = c & 1;
    const int l = (row & 31) + 32 * b;
    const int sig = l ^ (2 * (s & 3) + b) ^ (8 * (l & 1));
    a.k = (8 * kb + s) * 1024 + 16 * sig;
  }
  {
    const int r8 = row & 7, db = c >> 2;
    const int slot = (c & 1) + 2 * (r8 & 3) + 8 * ((c & 3) >> 1) + 16 * (r8 >> 2);
    const int sig = slot ^ (2 * ((c & 3) >> 1)) ^ (4 * (db & 1));
    const int id =
        ((2 * (row >> 5) + ((row >> 4) & 1)) * 4 + db) * 2 + ((row >> 3) & 1);
    a.v = 512 * id + 16 * sig;
  }
  return a;
}

// The 64 bytes one lane moves per step: chunks c and 8 + c (c = lane % 8) of
// its K row and of its V row.
struct Staged {
  uint4 k0, k1, v0, v1;
};

__device__ __forceinline__ Staged load_rows(const uint16_t* kbase,
                                            const uint16_t* vbase, int key,
                                            int nkeys, int lane) {
  key = min(max(key, 0), nkeys - 1);  // memory-safe for any indices
  const size_t off = (size_t)key * kHeadDim + 8 * (lane & 7);
  Staged r;
  r.k0 = *reinterpret_cast<const uint4*>(kbase + off);
  r.k1 = *reinterpret_cast<const uint4*>(kbase + off + 64);
  r.v0 = *reinterpret_cast<const uint4*>(vbase + off);
  r.v1 = *reinterpret_cast<const uint4*>(vbase + off + 64);
  return r;
}

__device__ __forceinline__ void store_rows(char* kdst, char* vdst,
                                           const Staged& r, StoreAddr a) {
  *reinterpret_cast<uint4*>(kdst + a.k) = r.k0;
  *reinterpret_cast<uint4*>(kdst + a.k + 4096) = r.k1;
  *reinterpret_cast<uint4*>(vdst + a.v) = r.v0;
  *reinterpret_cast<uint4*>(vdst + a.v + 2048) = r.v1;
}

// One lane's 32 bytes of one K or V row (chunks c and 8 + c).
struct Half {
  uint4 a, b;
};
__device__ __forceinline__ Half load_half(const uint16_t* base, int key,
                                          int nkeys, int lane) {
  key = min(max(key, 0), nkeys - 1);
  const size_t off = (size_t)key * kHeadDim + 8 * (lane & 7);
  Half r;
  r.a = *reinterpret_cast<const uint4*>(base + off);
  r.b = *reinterpret_cast<const uint4*>(base + off + 64);
  return r;
}
__device__ __forceinline__ void store_khalf(char* kdst, const Half& r,
                                            StoreAddr a) {
  *reinterpret_cast<uint4*>(kdst + a.k) = r.a;
  *reinterpret_cast<uint4*>(kdst + a.k + 4096) = r.b;
}
__device__ __forceinline__ void store_vhalf(char* vdst, const Half& r,
                                            StoreAddr a) {
  *reinterpret_cast<uint4*>(vdst + a.v) = r.a;
  *reinterpret_cast<uint4*>(vdst + a.v + 2048) = r.b;
}

// Per-lane read offsets of the swizzled layouts: K block (kb, s) is read at
// 1024 (8 kb + s) + kofs[s % 4]; V block id (column block db) at
// 512 id + vofs[db % 2].
struct ReadAddr {
  int kofs[4];
  int vofs[2];
};
__device__ __forceinline__ ReadAddr read_addr(int lane) {
  ReadAddr a;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    a.kofs[j] = 16 * (lane ^ (2 * j + (lane >> 5)) ^ (8 * (lane & 1)));
#pragma unroll
  for (int x = 0; x < 2; ++x)
    a.vofs[x] =
        16 * ((lane >> 1) ^ (2 * ((lane >> 4) & 1)) ^ (4 * x)) + 8 * (lane & 1);
  return a;
}

// S^T[kb]: keys kb*32 + 8(r/4) + 4 lh + r%4, query = the lane's row lane%32.
__device__ __forceinline__ void qk_tile(const char* Kt, const bf16x8 (&qr)[8],
                                        f32x16 (&sacc)[2], const ReadAddr& ra) {
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
  bf16x8 op[2][2];
  auto load = [&](int s, bf16x8 (&o)[2]) {
    const char* p = Kt + s * 1024 + ra.kofs[s & 3];
    o[0] = *reinterpret_cast<const bf16x8*>(p);
    o[1] = *reinterpret_cast<const bf16x8*>(p + 8 * 1024);
  };
  load(0, op[0]);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) load(s + 1, op[(s + 1) & 1]);
    sacc[0] = mfma32(op[s & 1][0], qr[s], sacc[0]);
    sacc[1] = mfma32(op[s & 1][1], qr[s], sacc[1]);
  }
}

__device__ __forceinline__ float lane_max(const f32x16 (&sacc)[2]) {
  float v4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) v4[r & 3] = fmaxf(v4[r & 3], sacc[kb][r]);
  return fmaxf(fmaxf(v4[0], v4[1]), fmaxf(v4[2], v4[3]));
}


// The online softmax of one tile in pieces (row max and rescale here, the
// exponentials in qk_exp, the PV product in pv_tile), so that the QK MFMAs
// of the next tile can be interleaved with the exponentials of this one.
// `active` false turns the step into a no-op with the same instructions:
// no rescale, every p = 0 (the reference is +inf), nothing added.
// Returns the reference the exponentials subtract.
__device__ __forceinline__ float row_rescale(const f32x16 (&sacc)[2],
                                             f32x16 (&oacc)[4], float& m,
                                             float& l, float c2, bool active) {
  float v = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[kb][r]);
  const float mx = max_xor32(v) * c2 + (active ? 0.f : -INFINITY);
  if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
    const float mnew = fmaxf(m, mx);
    const float alpha = m == mnew ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    m = mnew;
  }
  return !active ? INFINITY : m == -INFINITY ? 0.f : m;
}

__device__ __forceinline__ void pv_tile(const char* Vt, const f32x16 (&sacc)[2],
                                        f32x16 (&oacc)[4], const ReadAddr& ra) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kb = s >> 1, half = s & 1;
    f16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (_Float16)sacc[kb][8 * half + e];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int id = ((2 * kb + half) * 4 + db) * 2;
      const char* p = Vt + id * 512 + ra.vofs[db & 1];
      const s16x4 lo = lds_read_tr16(p);
      const s16x4 hi = lds_read_tr16(p + 512);
      const s16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = mfma32(__builtin_bit_cast(f16x8, cat), pb, oacc[db]);
    }
  }
}

// The QK of the next tile (into nxs) interleaved with the exponentials of
// this one (cur, in place): per k-step 2 MFMAs and 4 exponentials, the K
// operands one k-step ahead. Returns the row sum of the new p.
__device__ __forceinline__ float qk_exp(const char* Kt, const bf16x8 (&qr)[8],
                                        f32x16 (&nxs)[2], f32x16 (&cur)[2],
                                        float c2, float muse,
                                        const ReadAddr& ra) {
  nxs[0] = f32x16{};
  nxs[1] = f32x16{};
  bf16x8 op[2][2];
  auto load = [&](int s, bf16x8 (&o)[2]) {
    const char* p = Kt + s * 1024 + ra.kofs[s & 3];
    o[0] = *reinterpret_cast<const bf16x8*>(p);
    o[1] = *reinterpret_cast<const bf16x8*>(p + 8 * 1024);
  };
  float rs = 0.f;
  load(0, op[0]);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) load(s + 1, op[(s + 1) & 1]);
    nxs[0] = mfma32(op[s & 1][0], qr[s], nxs[0]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int x = 4 * s + e, kb = x >> 4, r = x & 15;
      const float p = __builtin_amdgcn_exp2f(cur[kb][r] * c2 - muse);
      cur[kb][r] = p;
      rs += p;
    }
    nxs[1] = mfma32(op[s & 1][1], qr[s], nxs[1]);
#pragma unroll
    for (int e = 2; e < 4; ++e) {
      const int x = 4 * s + e, kb = x >> 4, r = x & 15;
      const float p = __builtin_amdgcn_exp2f(cur[kb][r] * c2 - muse);
      cur[kb][r] = p;
      rs += p;
    }
  }
  return rs;
}

// s_waitcnt lgkmcnt(0) (gfx9 encoding; vmcnt and expcnt left unlimited)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Seven instances. kLocal: the local pass (every block's dense local window,
// rows in their own order); kLocalPair: the same with two blocks per
// workgroup, one after the other (see the mapping below; used where the four
// blocks of a workgroup share their heads and a segment's blocks pair up).
// kMaxRef and kFastRef: the sparse pass over the
// first n_I tiles of L_t, n_I given (the early stop's stop points or a
// budget). kFastRef raises the online softmax's reference only when p
// values grow past 2^8; it runs the workgroups whose logits are provably
// bounded, exits from the others and flags them for the kMaxRef launch that
// follows, which takes the row maximum of every tile and skips the
// unflagged workgroups. kExactMax: the sparse pass with the exact per-block
// max test deciding every tile of L_t in the loop. Workgroups of the sparse
// instances with no tile to visit exit at once: the local pass's output is
// final for their rows.
// kTopKMax and kTopKFast: the sparse pass over the per-block Top-K
// selections (a bitmask over the positions of L_t per block): the workgroup
// steps through the union of its blocks' selected positions, and a wave
// whose block did not select a position runs that step as a no-op (both
// halves of a block share a SIMD, so skipping the work would not shorten
// the step, which waits for the busiest SIMD); the two reference paths as
// for kMaxRef / kFastRef.
enum : int {
  kMaxRef = 0, kFastRef = 1, kExactMax = 2, kLocal = 3, kTopKMax = 4,
  kTopKFast = 5, kLocalPair = 6
};

template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fwd(AttnArgs a) {
  constexpr bool kExact = kMode == kExactMax;
  constexpr bool kTopK = kMode == kTopKMax || kMode == kTopKFast;
  constexpr bool kFast = kMode == kFastRef || kMode == kTopKFast;
  // kLocalPair: the local pass with two query blocks per workgroup, one
  // after the other: block i and block S / 64 - 1 - i of the same four heads
  // (S / 64 + 1 steps in all, the same for every workgroup); the key tiles
  // run on through both, and at the switch the first block's result is
  // written and the second block's queries are loaded
  constexpr bool kPair = kMode == kLocalPair;
  constexpr bool kLoc = kMode == kLocal || kPair;
  if ((kMode == kMaxRef || kMode == kTopKMax) && a.wg_flag[blockIdx.x] == 0)
    return;  // done
  // rings of four K and four V tile buffers of 16 KB (tile j in slot j % 4)
  __shared__ __attribute__((aligned(1024))) char kring[4][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vring[4][kTileBytes];
  __shared__ int wave_maxrow[kWaves];
  __shared__ int wave_ntiles[kWaves];
  // exact mode: each wave's maximum of the next tile, by step parity
  __shared__ unsigned tile_max[2][kWaves];
  // Top-K mode: the four blocks' masks, the union of their selected
  // positions (in L_t order) and, per step, which of the blocks take it
  // (per step: position | blocks << 16)
  __shared__ uint32_t tk_words[4][kMaskWords];
  __shared__ int tk_step[kMaxTiles];
  __shared__ int tk_count;
  __shared__ int pool_claim;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lh = lane >> 5;
  const int qsub = wave & 3, half = wave >> 2;

  // ---- which (b, g, t) group and which 4 query blocks.
  // Groups are ranked by descending t (longest work first). Consecutive
  // workgroup ids are dispatched round-robin over the 8 XCDs; group q runs on
  // XCD q % 8 so that all workgroups of one group share that XCD's L2.
  // Tail pool of the bounded-reference launch: the XCDs' shares of the work
  // differ (each holds the groups of its own KV heads, whose stop points
  // differ, and the XCDs do not run at quite the same speed), so the last
  // groups of every XCD's list go to a pool. A workgroup of a pool slot,
  // and each of the extra workgroups launched after the grid, claims the
  // next job of the pool (whole groups in list order, so a group's
  // workgroups mostly run together on one XCD and share its L2); the XCDs
  // that reach their pool slots first take more of it, and a workgroup
  // that finds the pool empty exits. The job (p) is then that slot.
  int p = blockIdx.x;
  if (kMode == kFastRef && a.pool_start >= 0 && (p >> 3) >= a.pool_start) {
    if (tid == 0) pool_claim = atomicAdd(a.pool_ctr, 1);
    __syncthreads();
    const int c = pool_claim;
    const int slots = (a.n_groups >> 3) * a.wg_per_group;
    if (c >= 8 * (slots - a.pool_start)) return;  // the pool is empty
    const int q = c / a.wg_per_group, ch = c % a.wg_per_group;
    p = (q & 7) +
        8 * ((a.pool_start / a.wg_per_group + (q >> 3)) * a.wg_per_group + ch);
  }
  // the local pass precedes every sparse pass: it clears the pool counter
  if (kLoc && blockIdx.x == 0 && tid == 0 && a.pool_ctr != nullptr)
    *a.pool_ctr = 0;
  int grp, chunk;
  if ((a.n_groups & 7) == 0) {
    const int x = p & 7, slot = p >> 3;
    grp = x + 8 * (slot / a.wg_per_group);
    chunk = slot % a.wg_per_group;
  } else {
    grp = p / a.wg_per_group;
    chunk = p % a.wg_per_group;
  }
  // local pass: the blocks nearest the segment's end (the most key tiles)
  // first; pairs: the workgroup's head quad and pair index pr give the
  // first block (S / 64 - 1 - pr, in the numbering of the one-block pass)
  // and the second (pr)
  int IbB = 0;
  if (kPair) {
    const int hq4 = a.G / 4, pr = chunk / hq4;
    IbB = pr;
    chunk = (a.S / kBlock - 1 - pr) * hq4 + chunk % hq4;
  } else if (kLoc) {
    chunk = a.wg_per_group - 1 - chunk;
  }
  const int BH = a.B * a.Hkv;
  const int t = a.T - 1 - grp / BH;
  const int bg = grp % BH, b = bg / a.Hkv, g = bg % a.Hkv;
  const int bps = a.S / kBlock;  // query blocks per segment and head
  const int seg0 = t * a.S;
  // query block e of the group: in order (local pass), or the sparse pass's
  // order by stop point
  const int ewg = chunk * 4 + qsub;
  const bool valid = ewg < a.G * bps;
  // Top-K: a workgroup's blocks are consecutive blocks of one head (neighbours
  // in pi_Q, whose selections overlap most)
  const int e = kTopK ? (valid ? (ewg % bps) * a.G + ewg / bps : ewg)
                : (!kLoc && a.border != nullptr && valid)
                    ? a.border[((long long)bg * a.T + t) * (a.G * bps) + ewg]
                    : ewg;

  // ---- the step sequence: the local pass's ndiag key blocks of the
  // segment, or the sparse passes' tiles of L_t up to the largest stop point
  // of the workgroup's blocks.
  const int ntl = t * bps;  // tiles of L_t
  const int32_t* Lt =
      a.L + (size_t)bg * a.list_len + (size_t)a.S * t * (t - 1) / 2;
  // sparse passes: no local step (the local pass covered those blocks);
  // a.local_steps is 0, read at run time as a value in [0, 1]: with a
  // literal 0 (or an unbounded value) the compiler schedules the loop with
  // more registers and spills
  const int ndiag_sparse = a.local_steps != 0 ? 1 : 0;

  // The first four tiles' rows are requested before the step count is
  // known (that takes a barrier): the local pass's tiles are the segment's
  // first key blocks, a sparse pass's the first tiles of L_t (indices
  // clamped into L_t; in the first segment, which has no L_t and no sparse
  // tile, an entry of pi_Q stands in as an in-bounds address). Rows of
  // steps beyond the count are loaded and never used. The index loads go
  // out with the block-order load, as neither depends on the other, and
  // branch-free, so that no wait for one sits between them; the row loads
  // go out before the wait for the block's pi_Q entries. That makes three
  // dependent memory round trips before the first tile (block order, pi_Q
  // entries, query rows; indices, key rows) where the plain order of the
  // statements made seven.
  const int rg = gather_row(wave, lane);
  if constexpr (kTopK) {
    // the union of the four blocks' selected positions, in L_t order
    const int hb = g * a.G + (valid ? e % a.G : 0);
    const size_t blk = ((size_t)b * a.Hq + hb) * (a.N / kBlock) + t * bps +
                       (valid ? e / a.G : 0);
    if (half == 0)
      tk_words[qsub][lane] = valid ? a.tmask[blk * kMaskWords + lane] : 0u;
    __syncthreads();
    if (wave == 0) {
      const uint32_t w0 = tk_words[0][lane], w1 = tk_words[1][lane],
                     w2 = tk_words[2][lane], w3 = tk_words[3][lane];
      uint32_t u = w0 | w1 | w2 | w3;
      const int cnt = __popc(u);
      int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int off = incl - cnt;
      while (u != 0u) {
        const int bit = __builtin_ctz(u);
        u &= u - 1u;
        const int blocks = (int)(((w0 >> bit) & 1u) | (((w1 >> bit) & 1u) << 1) |
                                 (((w2 >> bit) & 1u) << 2) |
                                 (((w3 >> bit) & 1u) << 3));
        tk_step[off] = (32 * lane + bit) | (blocks << 16);
        ++off;
      }
      if (lane == 63) tk_count = incl;
    }
    __syncthreads();
  }
  // Top-K: position of L_t that step s visits and the blocks that take it
  // (wave-uniform; past the last step: the last step's, in bounds)
  auto tk_entry = [&](int s) -> int {
    return __builtin_amdgcn_readfirstlane(
        tk_step[min(s, max(tk_count - 1, 0))]);
  };
  auto tk_position = [&](int s) -> int {
    return min(tk_entry(s) & 0xffff, max(ntl - 1, 0));
  };
  // local pass: the key block of step s (pairs: the second block's steps
  // start over at key block 0)
  const int IbA = kPair ? (chunk * 4) / a.G : 0;
  auto loc_block = [&](int s) {
    return kPair ? (s <= IbA ? s : s - IbA - 1) : s;
  };
  auto first_key = [&](int s) -> int {
    const bool computed = kLoc || s < ndiag_sparse || ntl == 0;
    const int k = kTopK ? tk_position(s)
                        : min(max(s - ndiag_sparse, 0), max(ntl - 1, 0));
    const int32_t* src = ntl == 0 ? a.pi_q + rg : Lt + (size_t)k * kBlock + rg;
    const int x = kLoc ? 0 : *src;
    return computed ? seg0 + loc_block(s) * kBlock + rg : x;
  };
  const int key0 = first_key(0), key1 = first_key(1), key2 = first_key(2),
            key3 = first_key(3);
  // indices of the rows step 0 loads: V rows of tile 3, K rows of tile 4
  int raw_v = kLoc ? 0 : key3;
  int raw_k = kLoc ? 0 : first_key(4);

  const int h = g * a.G + (valid ? e % a.G : 0);
  const int Ib = valid ? e / a.G : 0;  // block index within the segment
  const int I = t * bps + Ib;
  const size_t bh = (size_t)b * a.Hq + h;
  const int32_t* pq = a.pi_q + bh * a.N + (size_t)I * kBlock;
  int32_t* nI_ptr = a.n_I + bh * (a.N / kBlock) + I;
  // sparse passes: unconditional, no wait for it until used; the local pass
  // reads nothing the planner writes (it may run beside the planner)
  const int nI_raw = (kLoc || kTopK) ? 0 : *nI_ptr;
  const int nI = (!valid || kLoc) ? 0
                 : kExact ? ntl
                 : kTopK  ? tk_count
                          : min(max(nI_raw, 0), ntl);
  // my row: the local pass takes the segment's rows in their own order,
  // the sparse passes the rows of block I of pi_Q
  const int iq = kLoc ? seg0 + Ib * kBlock + 32 * half + lq
                      : min(max(pq[32 * half + lq], 0), a.N - 1);
  const int iqB = seg0 + IbB * kBlock + 32 * half + lq;  // pairs
  const uint16_t* qh = a.q + bh * a.N * kHeadDim;
  const uint16_t* kbase = a.k + (size_t)bg * a.N * kHeadDim;
  const uint16_t* vbase = a.v + (size_t)bg * a.N * kHeadDim;
  const StoreAddr sta = store_addr(rg, lane);
  const ReadAddr ra = read_addr(lane);
  const Staged r0 = load_rows(kbase, vbase, key0, a.N, lane);
  const Staged r1 = load_rows(kbase, vbase, key1, a.N, lane);
  const Staged r2 = load_rows(kbase, vbase, key2, a.N, lane);
  // staged for step 0's stores: K rows of tile 3, V rows of tile 2
  Half kst = load_half(kbase, key3, a.N, lane);
  Half vst = {r2.v0, r2.v1};

  // the lane's query row as Q^T B operands, for the whole run
  bf16x8 qr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qr[s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)iq * kHeadDim +
                                             16 * s + 8 * lh);

  // The local pass starts from nothing; the sparse passes continue the
  // online softmax of the local pass, whose normalised output (the bf16
  // value in O plus its bf16 residual) and log2-sum-exp are the state
  // o = acc / l, l = 1 for reference m = log2-sum-exp.
  f32x16 oacc[4];
  float m = -INFINITY, l = 0.f;
  if (kLoc) {
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  } else {
    const size_t ro = (bh * a.N + iq) * kHeadDim;
    float amax = 0.f;  // largest |value| of the lane's 64 bf16 values
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const size_t e = ro + db * 32 + 8 * g4 + 4 * lh;
        const uint2 w = *reinterpret_cast<const uint2*>(a.o + e);
        oacc[db][4 * g4 + 0] = __uint_as_float(w.x << 16);
        oacc[db][4 * g4 + 1] = __uint_as_float(w.x & 0xffff0000u);
        oacc[db][4 * g4 + 2] = __uint_as_float(w.y << 16);
        oacc[db][4 * g4 + 3] = __uint_as_float(w.y & 0xffff0000u);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          amax = fmaxf(amax, fabsf(oacc[db][4 * g4 + j]));
      }
    if (amax >= kResidualFrom) {  // the local pass stored the residuals
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const uint2 r = *reinterpret_cast<const uint2*>(
              a.olo + ro + db * 32 + 8 * g4 + 4 * lh);
          oacc[db][4 * g4 + 0] += __uint_as_float(r.x << 16);
          oacc[db][4 * g4 + 1] += __uint_as_float(r.x & 0xffff0000u);
          oacc[db][4 * g4 + 2] += __uint_as_float(r.y << 16);
          oacc[db][4 * g4 + 3] += __uint_as_float(r.y & 0xffff0000u);
        }
    }
    m = a.lse2[bh * a.N + iq];
    l = 1.f;
  }

  const int myrow = wave_max_int(iq);
  if (lane == 0) {
    wave_maxrow[wave] = valid ? myrow : -1;
    wave_ntiles[wave] = nI;
  }
  __syncthreads();
  int wgmax = -1, ntiles = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wgmax = max(wgmax, wave_maxrow[w]);
    ntiles = max(ntiles, wave_ntiles[w]);
  }
  const int ndiag = kPair  ? bps + 1
                    : kLoc ? min(max((wgmax - seg0) / kBlock + 1, 1), bps)
                           : ndiag_sparse;
  const int nsteps = ndiag + ntiles;
  if (!kLoc && ntiles == 0) {
    // no sparse tile: the local pass's output and lse are final
    if (kFast && tid == 0) a.wg_flag[p] = 0;
    if (kExact && valid && lane == 0 && half == 0) *nI_ptr = 0;
    __builtin_amdgcn_s_waitcnt(0);  // the first tiles' loads
    return;
  }

  // Tile indices: step s of a sparse pass loads the index of the row this
  // lane fetches for tile s + 4 (steps past the last one load a harmless
  // in-bounds value); the local pass computes its indices.
  auto key_src = [&](int s, int row) -> const int32_t* {
    if (kTopK)
      return s < nsteps ? Lt + (size_t)tk_position(s) * kBlock + row
                        : pq + (row & 63);
    return (s >= ndiag && s < nsteps) ? Lt + (size_t)(s - ndiag) * kBlock + row
                                      : pq + (row & 63);
  };
  auto key_of = [&](int s, int row, int raw) {
    return s < ndiag ? seg0 + loc_block(s) * kBlock + row : raw;
  };

  // Software pipeline, one step per tile s: the QK of tile s + 1 (K slot
  // (s + 1) % 4) is issued between the row rescale and the exponentials of
  // tile s, then the PV of tile s (V slot s % 4), then the staged K rows of
  // tile s + 3 and V rows of tile s + 2 go to their slots and the next rows
  // and indices are loaded. A barrier after every odd step (after every
  // step in the exact mode, whose maxima travel through LDS from one step
  // to the next). A wave whose block has stopped (or whose tile the exact
  // test rejects) runs the same instructions as a no-op. Before the first
  // step: K and V of tiles 0 and 1 and K of tile 2 in LDS, K of tile 3 and
  // V of tile 2 staged.
  store_rows(kring[0], vring[0], r0, sta);
  store_rows(kring[1], vring[1], r1, sta);
  store_khalf(kring[2], Half{r2.k0, r2.k1}, sta);
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk_tile(kring[0], qr, sa, ra);
  // the first pair of steps refills the slot of tile 0: every wave must have
  // read it (the bounded-row test and the exact mode's maxima end in a
  // barrier of their own)
  if (!kFast && !kExact) __syncthreads();
  // causal mask of a local step over keys j0 ..: key j0 + off of the tile is
  // masked iff off > iq - j0 - 4 lh (row iqx)
  auto mask_local = [&](int j0, int iqx, f32x16 (&cur)[2]) {
    const int lim = iqx - j0 - 4 * lh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
        cur[kb][r] = off > lim ? -INFINITY : cur[kb][r];
      }
  };
  float my_max = 0.f;  // exact mode: this half's maximum of the current tile
  if (kExact) {
    // tile 0's maxima for the exact test of step 0
    my_max = wave_max(lane_max(sa));
    if (lane == 0) tile_max[0][wave] = __float_as_uint(my_max);
    __syncthreads();
  }
  if (kFast) {
    // The logits of a row are bounded by |q| max_j |k_j| (Cauchy-Schwarz);
    // within kSafeSpan of the reference no p overflows before the rescale
    // test. A workgroup with an unbounded row leaves it to kMaxRef.
    float qn = 0.f;  // |q|^2 of the row, fp32
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qr[s][e];
        qn = fmaf(x, x, qn);
      }
    qn = sum_xor32(qn);
    // fp32 rounding of both norms and of the MFMA sums: a 2^-10 margin
    const float bound = sqrtf(qn * a.kmax2[bg]) * a.c2 * (1.f + 1.f / 1024.f);
    const bool safe = bound - m <= kSafeSpan;  // false for NaN
    const int unsafe = __syncthreads_or(valid && !safe);
    if (tid == 0) a.wg_flag[p] = unsafe;
    if (unsafe) {
      __builtin_amdgcn_s_waitcnt(0);  // loads issued by the prologue
      return;
    }
  }
  int n_visit = 0;     // exact mode: tiles attended
  auto body = [&](int s, f32x16 (&cur)[2], f32x16 (&nxs)[2], bool bar) {
    const bool local = s < ndiag;  // every step of the local pass
    // the local pass: block Ib sees key blocks 0 .. Ib, the last one masked
    // (pairs: the second block's last step is the workgroup's last)
    if (kLoc && s == Ib) mask_local(seg0 + Ib * kBlock, iq, cur);
    if (kPair && s == nsteps - 1) mask_local(seg0 + IbB * kBlock, iqB, cur);
    bool act = valid && (kPair   ? true
                         : kLoc  ? s <= Ib
                         : kTopK ? ((tk_entry(s) >> (16 + qsub)) & 1) != 0
                                 : (s - ndiag) < nI);
    if (kExact && !local) {
      // exact max test of tile s: both halves take max(own, other) of the
      // maxima posted with the tile's logits, before the last barrier
      const float other = __uint_as_float(tile_max[s & 1][wave ^ 4]);
      const bool take = fmaxf(my_max, other) >= a.exact_thr;
      n_visit += (act && take) ? 1 : 0;
      act = act && take;
    }
    if (kExact && !act) {
      // a tile the exact test rejects (most of them): only the next QK
      qk_tile(kring[(s + 1) & 3], qr, nxs, ra);
    } else {
      const float muse = kFast ? (act ? m : INFINITY)
                               : row_rescale(cur, oacc, m, l, a.c2, act);
      __builtin_amdgcn_sched_barrier(0);
      float rs = qk_exp(kring[(s + 1) & 3], qr, nxs, cur, a.c2, muse, ra);
      if (kFast && __builtin_amdgcn_ballot_w64(rs > kRescaleSum) != 0) {
        // rare: a p value may exceed 2^8; divide the row by its largest p
        // (this raises the reference by log2 of it)
        const float pm = max_xor32(lane_max(cur));
        if (pm > 1.f) {
          const float sc = __builtin_amdgcn_rcpf(pm);
          m += __builtin_amdgcn_logf(pm);
          l *= sc;
          rs *= sc;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) cur[kb] *= sc;
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[db] *= sc;
        }
      }
      l += sum_xor32(rs);
      __builtin_amdgcn_sched_barrier(0);
      pv_tile(vring[s & 3], cur, oacc, ra);
    }
    if (kExact) {
      // this half's maximum of tile s + 1, for the other half (the slot of
      // step s + 1's parity; the other slot is being read this step)
      my_max = wave_max(lane_max(nxs));
      if (lane == 0) tile_max[(s + 1) & 1][wave] = __float_as_uint(my_max);
    }
    // K rows of tile s + 3 and V rows of tile s + 2 (loaded during step
    // s - 1) into the slots of tiles s - 1 and s - 2, then the loads of the
    // K rows of tile s + 4, the V rows of tile s + 3 and the index of tile
    // s + 5
    store_khalf(kring[(s + 3) & 3], kst, sta);
    store_vhalf(vring[(s + 2) & 3], vst, sta);
    vst = load_half(vbase, key_of(s + 3, rg, raw_v), a.N, lane);
    kst = load_half(kbase, key_of(s + 4, rg, raw_k), a.N, lane);
    raw_v = raw_k;
    if (!kLoc) raw_k = *key_src(s + 5, rg);
    if (bar) {
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
  };
  // ---- epilogue of row iqx: normalise, round to bf16, scatter to the
  // original row (the local pass also stores each value's residual below
  // its bf16 value, for the sparse pass to resume from).
  auto finish = [&](int iqx) {
    const float ln2 = 0.69314718055994530942f;
    const float inv = 1.f / l;
    const size_t ro = (bh * a.N + iqx) * kHeadDim;
    uint2 res[16];     // local pass: the residuals of the lane's 64 values
    float amax = 0.f;  // and the largest |bf16 value| among them
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * lh;
        __bf16 v4[4], r4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = oacc[db][4 * g4 + j] * inv;
          v4[j] = (__bf16)y;
          if (kLoc) {
            r4[j] = (__bf16)(y - (float)v4[j]);  // exact difference
            amax = fmaxf(amax, fabsf((float)v4[j]));
          }
        }
        *reinterpret_cast<uint2*>(a.o + ro + d0) =
            __builtin_bit_cast(uint2, v4);
        if (kLoc) res[4 * db + g4] = __builtin_bit_cast(uint2, r4);
      }
    // residuals only where they matter: values below kResidualFrom in
    // magnitude lose at most 2^-9 of it by the rounding to bf16, well inside
    // the output tolerance; the sparse pass reads them under the same test
    // on the same bf16 values
    if (kLoc && amax >= kResidualFrom) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint2*>(a.olo + ro + db * 32 + 8 * g4 + 4 * lh) =
              res[4 * db + g4];
    }
    const float lse2v = m + log2f(l);
    if (kLoc && lh == 0) a.lse2[bh * a.N + iqx] = lse2v;
    if (a.lse != nullptr && lh == 0) a.lse[bh * a.N + iqx] = lse2v * ln2;
  };

  // steps of the first (or only) block
  const int nfirst = kPair ? IbA + 1 : nsteps;
  int s = 0;
  for (; s + 1 < nfirst; s += 2) {
    body(s, sa, sb, kExact);
    body(s + 1, sb, sa, true);
  }
  if (s < nfirst) body(s, sa, sb, false);
  if constexpr (kPair) {
    // the switch: the first block's result out, the softmax restarted for
    // the second block's rows and its first tile's QK recomputed with their
    // queries (the last step computed it with the first block's); the key
    // tiles in flight are already the second block's
    __builtin_amdgcn_s_waitcnt(0);
    finish(iq);
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x)
      qr[x] = *reinterpret_cast<const bf16x8*>(qh + (size_t)iqB * kHeadDim +
                                               16 * x + 8 * lh);
    qk_tile(kring[nfirst & 3], qr, sa, ra);
    // every wave has read that tile before any refills its slot (the pair
    // of steps that starts with an even first step of the second block
    // writes it)
    __syncthreads();
    s = nfirst;
    // a barrier after every odd step, as before the switch
    for (; s + 1 < nsteps; s += 2) {
      body(s, sa, sb, (s & 1) != 0);
      body(s + 1, sb, sa, (s & 1) == 0);
    }
    if (s < nsteps) body(s, sa, sb, false);
  }
  __builtin_amdgcn_s_waitcnt(0);  // index loads of steps never taken

  if (!valid) return;
  finish(kPair ? iqB : iq);
  if (kExact && lane == 0 && half == 0) *nI_ptr = n_visit;
}

// V in fp16 for the PV products: each bf16 value (8 bits of significand) is
// exactly an fp16 value when its magnitude lies in fp16's normal range
// [2^-14, 65504]; smaller ones round to fp16's subnormal steps of 2^-24,
// larger ones overflow. One thread per 8 values (16-byte loads and stores).
__global__ __launch_bounds__(256) void k_v_to_f16(const uint4* __restrict__ v,
                                                  uint4* __restrict__ v16,
                                                  long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 w = v[i];
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 r;
    r[0] = (_Float16)__uint_as_float(in[j] << 16);
    r[1] = (_Float16)__uint_as_float(in[j] & 0xffff0000u);
    out[j] = __builtin_bit_cast(uint32_t, r);
  }
  v16[i] = make_uint4(out[0], out[1], out[2], out[3]);
}

int attention_blocks_per_wg() { return 4; }

void set_tail_pool(AttnArgs& a) {
  // the last 8 groups of each XCD's list (at most all of them), with up to
  // half as many extra workgroups per XCD as it has pool slots
  a.pool_start = -1;
  a.pool_extra = 0;
  if ((a.n_groups & 7) != 0 || a.n_groups < 8) return;
  const int per_xcd = a.n_groups >> 3;
  const int pg = per_xcd < 8 ? per_xcd : 8;
  a.pool_start = (per_xcd - pg) * a.wg_per_group;
  a.pool_extra = pg * a.wg_per_group / 2;
}

hipError_t launch_attention_local(const AttnArgs& a, hipStream_t s) {
  const long long n8 = (long long)a.B * a.Hkv * a.N * (kHeadDim / 8);
  hipLaunchKernelGGL(k_v_to_f16, dim3((unsigned)((n8 + 255) / 256)),
                     dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(a.v_in),
                     reinterpret_cast<uint4*>(a.v16), n8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the dense local windows in the rows' own order; two blocks per
  // workgroup when the four blocks of a workgroup share their heads (G a
  // multiple of 4) and the blocks of a segment pair up (an even count)
  const int bps = a.S / kBlock;
  if (a.G % 4 == 0 && bps % 2 == 0) {
    AttnArgs ap = a;
    ap.wg_per_group = a.wg_per_group / 2;
    const int total = a.n_groups * ap.wg_per_group;
    hipLaunchKernelGGL(k_attn_fwd<kLocalPair>, dim3(total), dim3(kThreads), 0,
                       s, ap);
    return hipGetLastError();
  }
  const int total = a.n_groups * a.wg_per_group;
  hipLaunchKernelGGL(k_attn_fwd<kLocal>, dim3(total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention_sparse(const AttnArgs& a, hipStream_t s) {
  if (a.local_only) return hipSuccess;
  const int total = a.n_groups * a.wg_per_group;
  if (a.exact) {
    hipLaunchKernelGGL(k_attn_fwd<kExactMax>, dim3(total), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
  }
  if (a.topk) {
    hipLaunchKernelGGL(k_attn_fwd<kTopKFast>, dim3(total), dim3(kThreads), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_fwd<kTopKMax>, dim3(total), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
  }
  // the bounded workgroups, then (flagged by the first launch) the others
  const int fast_total =
      total + (a.pool_start >= 0 ? 8 * a.pool_extra : 0);
  hipLaunchKernelGGL(k_attn_fwd<kFastRef>, dim3(fast_total), dim3(kThreads),
                     0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_fwd<kMaxRef>, dim3(total), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace sa
