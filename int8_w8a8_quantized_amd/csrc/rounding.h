// Exact rint(fl(x / s)) for whole arrays of values that share one scale, by
// multiplication: the integer codes of the activation quantiser and of the
// FP8 -> int8 weight conversion. Both rules divide a float by a float scale
// and round half to even ("[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴",
// 핵심 코드 분석 §3; "MiniMax-M2.7 FP8 转昆仑芯 INT8", 转换关系).
//
// The division is replaced by t = fl(x * r) with r = fl(1 / s). Whenever 1/s
// is a normal number, |t - fl(x/s)| < |t| * 2^-22 (two roundings of relative
// size 2^-24 in t, one in fl(x/s)). t is clamped to the code range L first
// (the bounds are integers, so clamping and rounding commute, and a clamped t
// saturates either way), so if t is farther than L * 2^-22 from every
// half-integer both round to the same integer. t is rounded by adding
// 1.5 * 2^23, which leaves rint(t) in the low mantissa bits (two's complement
// in the low byte). A group with a value near a half-integer, and a scale
// outside (2^-100, 2^100), takes the true division.
#pragma once

#include "device_common.h"

namespace w8a8 {

struct RowParams {
  float s;     // scale
  float r;     // fl(1/s)
  int zp;      // zero point (0 for symmetric rules)
  bool fast;   // 1/s is comfortably normal: the multiply-and-check path applies
};

__device__ __forceinline__ RowParams finish_params(float s, int zp) {
  RowParams p;
  p.s = s;
  p.zp = zp;
  p.fast = s > 0x1p-100f && s < 0x1p100f;
  p.r = 1.0f / s;
  return p;
}

// Adding kMagic = 1.5 * 2^23 to a float of magnitude <= 2^22 rounds it to an
// integer (ties to even) and leaves that integer + 0x400000 in the mantissa.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

// m[e] = bits of clamp(rint(fl(x[e] / s)), -L, L) + kMagic: the integer is
// m[e] - kMagicBits, and its low byte is the int8 code when |integer| <= 127.
// CLAMP = false: the caller guarantees s = fl(amax / L) with amax >= |x[e]|
// for every e. Then |fl(x * fl(1/s))| <= L * (1 + 2^-24)^3 < L + 1/2, so the
// clamp cannot change the result and is left out (scales outside the fast
// range still take the clamped true division).
template <int NV, int L, bool CLAMP = true>
__device__ __forceinline__ void round_quotients(const float* x, const RowParams& p, uint32_t* m) {
  constexpr float kLim = (float)L;
  constexpr float kTie = 0.5f - kLim * 0x1p-22f;  // |t| <= L: t, fl(x/s) differ by < L * 2^-22
  bool fix = !p.fast;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const float t = CLAMP ? fminf(fmaxf(x[e] * p.r, -kLim), kLim) : x[e] * p.r;
    const float r = t + kMagic;
    fix |= fabsf(t - (r - kMagic)) >= kTie;
    m[e] = __float_as_uint(r);
  }
  if (__builtin_expect(fix, 0)) {
#pragma unroll
    for (int e = 0; e < NV; ++e) m[e] = __float_as_uint(fminf(fmaxf(rne(x[e] / p.s), -kLim), kLim) + kMagic);
  }
}

// Low bytes of four words packed into one (v_perm_b32).
__device__ __forceinline__ uint32_t low_bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

}  // namespace w8a8
