// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_launch.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Fixed-point image used by every ranking score: round-half-even of 256 x,
// saturated to the int16 range. 256 x is exact in fp32 for a bfloat16 x.
__device__ __forceinline__ int32_t fixed_point(uint32_t bits16) {
  float x = rintf(bf16_bits_to_f32(bits16) * 256.0f);
  x = fminf(fmaxf(x, -32768.0f), 32767.0f);
  return (int32_t)x;
}

// The 8 fixed-point values of 8 packed bfloat16 (one 16-byte load).
__device__ __forceinline__ void fixed_point8(uint4 w, int32_t (&f)[8]) {
  f[0] = fixed_point(w.x & 0xffffu); f[1] = fixed_point(w.x >> 16);
  f[2] = fixed_point(w.y & 0xffffu); f[3] = fixed_point(w.y >> 16);
  f[4] = fixed_point(w.z & 0xffffu); f[5] = fixed_point(w.z >> 16);
  f[6] = fixed_point(w.w & 0xffffu); f[7] = fixed_point(w.w >> 16);
}

__device__ __forceinline__ int64_t shfl_xor_i64(int64_t v, int mask) {
  int lo = (int)(uint32_t)(uint64_t)v;
  int hi = (int)(uint32_t)((uint64_t)v >> 32);
  lo = __shfl_xor(lo, mask);
  hi = __shfl_xor(hi, mask);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over the 16 lanes of an aligned 16-lane group.
__device__ __forceinline__ int64_t sum16_i64(int64_t v) {
  v += shfl_xor_i64(v, 8);
  v += shfl_xor_i64(v, 4);
  v += shfl_xor_i64(v, 2);
  v += shfl_xor_i64(v, 1);
  return v;
}

// Ascending sort key for "score descending": order-preserving map of the
// signed score to unsigned, then complemented.
__device__ __forceinline__ uint64_t desc_key(int64_t score) {
  return ~((uint64_t)score ^ 0x8000000000000000ull);
}

__device__ __forceinline__ bool pair_less(uint64_t ka, int32_t ia,
                                          uint64_t kb, int32_t ib) {
  return ka < kb || (ka == kb && ia < ib);
}

}  // namespace sa
