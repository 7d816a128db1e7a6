// Exact rint(fl(x / s)) for whole arrays of values that share one scale, by
// multiplication: the integer codes of the activation quantiser and of the
// FP8 -> int8 weight conversion. Both rules divide a float by a float scale
// and round half to even ("[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴",
// 핵심 코드 분석 §3; "MiniMax-M2.7 FP8 转昆仑芯 INT8", 转换关系).
//
// The division is replaced by the product with r = fl(1 / s). A float of
// magnitude <= 2^22 added to c = 1.5 * 2^23 + z (z a small integer) rounds to
// an integer and leaves n + z in the low mantissa bits of the sum, n the
// nearest integer to the addend (two's complement in the low byte): the code
// with its zero point comes out of one addition. The result is the exact
// rint(fl(x/s)) whenever the value being rounded is not within
// L * 2^-22 + 2^-24 of a half-integer, L bounding |x/s|: the product differs
// from fl(x/s) by less than L * 2^-23 (one rounding in r, one in the quotient),
// the measured distance is itself rounded once (2^-25). Each group of values
// checks that distance; a group with a value near a half-integer, or a scale
// outside (2^-100, 2^100), takes the true division.
//
// Two forms:
//  - bounded (CLAMP = false), for scales derived from the values themselves
//    (s = fl(amax / 127), or fl((max - min) / 255) with the zero point of the
//    minimum): every x/s lies within 1 of [lo, hi], so no clamp is needed and
//    the product and rounding fuse: n from fma(x, r, c), the distance from
//    fma(x, r, c - sum) (exact product, one rounding; c - sum = -n exactly).
//  - clamped (CLAMP = true), for a given scale: t = fl(x r) is first clamped
//    to the integer range [lo, hi] of the codes before the zero point
//    (clamping and rounding commute for integer bounds, and a clamped t
//    saturates either way), so every sum lands in the code range.
#pragma once

#include "device_common.h"

namespace w8a8 {

// Adding kMagic = 1.5 * 2^23 to a float of magnitude <= 2^22 rounds it to an
// integer (ties to even) and leaves that integer + 0x400000 in the mantissa.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

struct RowParams {
  float s;       // scale
  float r;       // fl(1/s)
  float c;       // kMagic + zero point
  float lo, hi;  // range of rint(x/s) that maps into the codes: [qmin - zp, qmax - zp]
  float tie;     // the fast path is exact while every |value - n| < tie
  int zp;        // zero point (0 for symmetric rules)
  bool fast;     // 1/s is comfortably normal: the multiply-and-check path applies
};

// lo, hi: integers with max(|lo|, |hi|) <= 2^21 (the tie margin below is then
// exact in binary32 and positive).
__device__ __forceinline__ RowParams finish_params(float s, int zp, float lo, float hi) {
  RowParams p;
  p.s = s;
  p.zp = zp;
  p.c = kMagic + (float)zp;
  p.lo = lo;
  p.hi = hi;
  p.tie = 0.5f - fmaxf(-lo, hi) * 0x1p-22f - 0x1p-24f;
  p.fast = s > 0x1p-100f && s < 0x1p100f;
  p.r = 1.0f / s;
  return p;
}

// m[e] = bits of p.c + n[e], n[e] = rint(fl(x[e] / s)) (clamped to [lo, hi]
// when CLAMP): the integer n[e] + zp is m[e] - kMagicBits, and its low byte
// is the int8 code when it lies in [-128, 127].
// CLAMP = false: the caller guarantees lo - 1 <= x[e] / s <= hi + 1 for every
// e (exact quotient); n[e] is not clamped and can then be one outside
// [lo, hi], which the caller clamps where the rule allows it.
template <int NV, bool CLAMP>
__device__ __forceinline__ void round_quotients(const float* x, const RowParams& p, uint32_t* m) {
  float dev = 0.0f;  // largest distance to the rounded integer
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    float sum, d;
    if (CLAMP) {
      const float t = fminf(fmaxf(x[e] * p.r, p.lo), p.hi);
      sum = t + p.c;
      d = t - (sum - p.c);
    } else {
      sum = fmaf(x[e], p.r, p.c);
      d = fmaf(x[e], p.r, p.c - sum);
    }
    dev = fmaxf(dev, fabsf(d));
    m[e] = __float_as_uint(sum);
  }
  if (__builtin_expect(!p.fast || !(dev < p.tie), 0)) {
#pragma unroll
    for (int e = 0; e < NV; ++e) m[e] = __float_as_uint(fminf(fmaxf(rne(x[e] / p.s), p.lo), p.hi) + p.c);
  }
}

// Low bytes of four words packed into one (v_perm_b32).
__device__ __forceinline__ uint32_t low_bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

}  // namespace w8a8
