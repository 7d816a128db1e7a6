// Pieces shared by the int8 GEMM kernels: the MFMA step and the fused
// scale / zero-point / bias epilogue of "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도
// 양자화 스킴" (핵심 코드 분석 §3-§4).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

// v_mfma_i32_16x16x64_i8: D[16x16] += A[16x64] * B[64x16], exact int32.
// Operand lane layout (both operands): lane l supplies row (A) / column (B)
// l % 16 and 16 consecutive k values of k-group l / 16. Only the pairing of
// A's and B's k-groups matters for a dot product, so any consistent k order
// gives the same exact sums. Result layout: lane l holds rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ i32x4 mfma16x16x64(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// v_mfma_i32_32x32x32_i8: D[32x32] += A[32x32] * B[32x32], exact int32, at
// twice the int8 rate of the 16x16x64 form on gfx950. Operand lane layout:
// lane l supplies row (A) / column (B) l % 32 and 16 consecutive k values of
// k-group l / 32 (the same pairing argument as above applies). Result
// layout: lane l holds column l % 32; its register r holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4.
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ i32x16 mfma32x32x32(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands with unit (E8M0 127)
// block scales: D[32x32] += A[32x64] * B[64x32] in binary32. Lane l supplies
// row (A) / column (B) l % 32 and 32 consecutive k values of k-group l / 32
// (any order consistent between A and B gives the same products); the
// accumulators have the 32x32x32 int8 layout and are kept as bit patterns.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ i32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, i32x16 c) {
  return __builtin_bit_cast(i32x16, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                         a, b, __builtin_bit_cast(f32x16, c), 0, 0, 0, 127, 0, 127));
}

__device__ __forceinline__ i32x4 as_i32x4(uint4 v) {
  i32x4 r;
  r.x = (int)v.x;
  r.y = (int)v.y;
  r.z = (int)v.z;
  r.w = (int)v.w;
  return r;
}

// Epilogue of one output element. c = acc - correction (exact int32), then
// bf16(float(c) * s_x * s_w + bias) or c itself.
struct EpiRow {
  float sx;
  int zp;   // per-token zero point (used only with AZP_PER_TOKEN)
  bool ok;  // row inside the output
  int64_t out_row;
};
struct EpiCol {
  float sw;
  int corr;            // colsum[n] (per-token AZP) or azp_adj[n] (static AZP); unused otherwise
  uint32_t bias_bits;  // bf16 bits of bias[n] (meaningless without bias), widened when used
  bool ok;
  __device__ __forceinline__ float bias() const { return __uint_as_float(bias_bits << 16); }
};

__device__ __forceinline__ void epilogue_store(const GemmArgs& a, const EpiRow& r, const EpiCol& c,
                                               int64_t col, int acc) {
  if (!(r.ok && c.ok)) return;
  int v = acc;
  if (a.azp_mode == 1) v -= r.zp * c.corr;
  else if (a.azp_mode == 2) v -= c.corr;
  if (a.out_i32) {
    reinterpret_cast<int32_t*>(a.out)[r.out_row * a.ldo + col] = v;
  } else {
    float y = (float)v * r.sx * c.sw;
    if (a.bias) y += c.bias();
    reinterpret_cast<uint16_t*>(a.out)[r.out_row * a.ldo + col] = f32_to_bf16_rne(y);
  }
}

__device__ __forceinline__ EpiCol load_col(const GemmArgs& a, int64_t n, const float* sw,
                                           const uint16_t* bias) {
  EpiCol c;
  c.ok = n < a.N;
  const int64_t nn = c.ok ? n : 0;
  // Addresses are selected instead of values (a missing operand reads the
  // scale, which always exists, and is never used), so no instruction next
  // to the loads consumes them and the wait for them lands at the epilogue.
  c.sw = sw[a.sw_per_channel ? nn : 0];
  c.corr = *(a.azp_mode != 0 ? a.colsum + nn : reinterpret_cast<const int32_t*>(sw));
  c.bias_bits = *(bias ? bias + nn : reinterpret_cast<const uint16_t*>(sw));
  return c;
}

}  // namespace w8a8
