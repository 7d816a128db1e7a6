// Device helpers shared by the gfx950 kernels of libw8a8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bits -> float: bf16 is the upper half of binary32, so this is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (finite and infinite inputs; a NaN
// input keeps a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> two bf16 packed in one word (low half = a), round to nearest
// even, by gfx950's v_cvt_pk_bf16_f32 (quiet NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round to nearest integer, ties to even (v_rndne_f32).
__device__ __forceinline__ float rne(float v) { return __builtin_rintf(v); }

// Wave-wide reductions over all 64 lanes (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Wave-wide IEEE-754 maximum / minimum without LDS traffic: within each row
// of 16 lanes by DPP moves (swap neighbours, swap pairs, half-row mirror, row
// mirror), then across the four rows by lane reads; every lane gets the
// result. NaN propagates.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ float wave_extreme(float v) {
  auto op = [](float a, float b) {
    return MAX ? __builtin_elementwise_maximum(a, b) : __builtin_elementwise_minimum(a, b);
  };
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror
  v = op(v, dpp_move<0x140>(v));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// 16-byte global load / store.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
// 16-byte load of data read exactly once (non-temporal: do not keep it in cache).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Sum of the four signed bytes of each of the four words (v_dot4_i32_i8 with ones).
__device__ __forceinline__ int sum_i8x16(uint4 v, int acc) {
  acc = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, acc, false);
  return acc;
}

// Pack four ints (already in [-128,127]) into one word of signed bytes.
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return min(max(v, lo), hi); }

}  // namespace w8a8
