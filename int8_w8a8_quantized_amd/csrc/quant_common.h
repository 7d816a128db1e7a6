// Per-chunk pieces of the activation quantiser shared by its kernels and by
// the decode GEMM that quantises its own activation rows: codes of 8 bf16
// values, the extremes of a chunk, and a row's rounding parameters from its
// extremes. The rules they follow are stated where quant.hip describes its
// kernels.
#pragma once

#include "device_common.h"
#include "rounding.h"

namespace w8a8 {

enum { kDynSym = 0, kDynAsym = 1, kStaticSym = 2, kStaticAsym = 3 };

// Codes of one 16-byte chunk (8 bf16) as 8 bytes.
template <int MODE>
__device__ __forceinline__ uint2 codes8(uint4 v, const RowParams& p) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float xs[8];
  uint32_t m[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xs[2 * i] = bf16_lo(w[i]);
    xs[2 * i + 1] = bf16_hi(w[i]);
  }
  // Dynamic scales come from the row's own extremes, so the quotients stay
  // within one of the code range and need no clamp before rounding; a given
  // (static) scale is clamped to [qmin - zp, qmax - zp] first.
  constexpr bool kDynamic = MODE == kDynSym || MODE == kDynAsym;
  round_quotients<8, !kDynamic>(xs, p, m);
  if (MODE == kDynAsym) {
    // the asymmetric quotients can round one past the top of the range
    // (x/s and min/s both just beyond a half-integer): clamp the biased
    // integer, whose low byte is the code
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = min(max(m[e], kMagicBits - 128u), kMagicBits + 127u);
  }
  uint2 o;
  o.x = low_bytes4(m[0], m[1], m[2], m[3]);
  o.y = low_bytes4(m[4], m[5], m[6], m[7]);
  return o;
}

// The extremes use IEEE-754 maximum / minimum (v_maximum3_f32 /
// v_minimum3_f32): they need no canonicalisation of their inputs, which the
// libm fmaxf / fminf would cost once per element; their NaN behaviour does
// not matter here, as non-finite activations are outside the contract.
__device__ __forceinline__ float max_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float min_ieee(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// Largest magnitude of one chunk folded into a.
__device__ __forceinline__ void absmax8(uint4 v, float& a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) a = max_ieee(a, max_ieee(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
}

__device__ __forceinline__ void minmax8(uint4 v, float& lo, float& hi) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
    lo = min_ieee(lo, min_ieee(a, b));
    hi = max_ieee(hi, max_ieee(a, b));
  }
}

// Row parameters from the reduced extremes. lo <= 0 <= hi always, since both
// start at 0 (the asymmetric range is widened to contain zero; for the
// symmetric mode absmax = max(hi, -lo)). The rounding range [lo, hi] of the
// quotients is the code range shifted by the zero point.
template <int MODE>
__device__ __forceinline__ RowParams row_params(float lo, float hi, const float* s_in,
                                                const int32_t* zp_in) {
  if (MODE == kDynSym) {
    const float a = fmaxf(hi, -lo);
    return finish_params((a == 0.0f) ? 1.0f : a / 127.0f, 0, -127.0f, 127.0f);
  }
  if (MODE == kDynAsym) {
    if (hi == lo) return finish_params(1.0f, 0, -128.0f, 127.0f);
    const float s = (hi - lo) / 255.0f;
    const float z = fminf(fmaxf(rne(lo / s), -512.0f), 512.0f);
    const int zp = clampi(-128 - (int)z, -128, 127);
    return finish_params(s, zp, (float)(-128 - zp), (float)(127 - zp));
  }
  if (MODE == kStaticSym) return finish_params(*s_in, 0, -127.0f, 127.0f);
  // a zero point of an int8 code range; beyond +-2^20 the shifted range would
  // leave the exact integers of the rounding (the contract asks for [-128, 127])
  const int zp = clampi(*zp_in, -(1 << 20), 1 << 20);
  return finish_params(*s_in, zp, (float)(-128 - zp), (float)(127 - zp));
}

}  // namespace w8a8
