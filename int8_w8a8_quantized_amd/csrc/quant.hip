// Activation quantisation kernels: bf16 rows -> int8 codes (+ per-token scale
// and zero point).
//
// Per-token symmetric: the per-row absmax/127 rule of "MiniMax-M2.7 FP8 转昆仑芯
// INT8" (转换关系) applied to each token row, as the per-token quantiser of
// "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴" (핵심 코드 분석 §3) uses it;
// asymmetric: the affine mapping with an int8 zero point that the same page
// (§3-§4) and "vLLM INT8 W8A8 量化实战" (4.2) describe; static: one calibrated
// scale (and zero point) for the whole tensor ("vLLM INT8 W8A8 量化实战" 4.1).
//
// One wave owns one row. The row is read once with 16-byte loads (8 bf16 per
// lane per chunk, consecutive lanes on consecutive chunks so each wave
// instruction moves 1 KiB of contiguous HBM) and kept in registers while the
// wave reduces its absmax (or min and max) with cross-lane shuffles; the codes
// are then written as 8-byte stores, again contiguous across the wave. HBM
// traffic is the algorithmic 2 B read + 1 B written per element. Rows longer
// than the register budget take a two-pass variant that re-reads the row
// (an L2 hit: one row is at most 128 KiB).
//
// Every float step is one IEEE binary32 operation: the absmax and min/max are
// exact, the scale is a true division by 127 (or 255), and each code is
// rint(x / s) with a true division and round-half-to-even, so the codes equal
// the exactly defined ones bit for bit.

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

enum { kDynSym = 0, kDynAsym = 1, kStaticSym = 2, kStaticAsym = 3 };

struct RowParams {
  float s;
  int zp;
};

// Code of one element. Symmetric: clamp(rint(x/s), -127, 127). Asymmetric:
// clamp(rint(x/s) + zp, -128, 127); the quotient is clamped to +-512 before the
// integer add, which cannot change the result since |zp| <= 128.
template <int MODE>
__device__ __forceinline__ int code_of(float x, RowParams p) {
  float r = rne(x / p.s);
  if (MODE == kDynSym || MODE == kStaticSym) {
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
  }
  r = fminf(fmaxf(r, -512.0f), 512.0f);
  return clampi((int)r + p.zp, -128, 127);
}

template <int MODE>
__device__ __forceinline__ uint2 codes8(uint4 v, RowParams p) {
  uint2 o;
  o.x = pack4(code_of<MODE>(bf16_lo(v.x), p), code_of<MODE>(bf16_hi(v.x), p),
              code_of<MODE>(bf16_lo(v.y), p), code_of<MODE>(bf16_hi(v.y), p));
  o.y = pack4(code_of<MODE>(bf16_lo(v.z), p), code_of<MODE>(bf16_hi(v.z), p),
              code_of<MODE>(bf16_lo(v.w), p), code_of<MODE>(bf16_hi(v.w), p));
  return o;
}

__device__ __forceinline__ void minmax8(uint4 v, float& lo, float& hi) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
    lo = fminf(lo, fminf(a, b));
    hi = fmaxf(hi, fmaxf(a, b));
  }
}

// Row parameters from the wave-reduced extremes. lo <= 0 <= hi always, since
// both start at 0 (the asymmetric range is widened to contain zero; for the
// symmetric mode absmax = max(hi, -lo)).
template <int MODE>
__device__ __forceinline__ RowParams row_params(float lo, float hi, const float* s_in,
                                                const int32_t* zp_in) {
  RowParams p;
  if (MODE == kDynSym) {
    float a = fmaxf(hi, -lo);
    p.s = (a == 0.0f) ? 1.0f : a / 127.0f;
    p.zp = 0;
  } else if (MODE == kDynAsym) {
    if (hi == lo) {
      p.s = 1.0f;
      p.zp = 0;
    } else {
      p.s = (hi - lo) / 255.0f;
      float z = fminf(fmaxf(rne(lo / p.s), -512.0f), 512.0f);
      p.zp = clampi(-128 - (int)z, -128, 127);
    }
  } else {
    p.s = *s_in;
    p.zp = (MODE == kStaticAsym) ? *zp_in : 0;
  }
  return p;
}

// CH = 16-byte chunks per lane held in registers; rows with K <= CH*512.
template <int MODE, int CH>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                         int64_t M, int64_t K, int64_t ldx,
                                                         const float* __restrict__ s_in,
                                                         const int32_t* __restrict__ zp_in,
                                                         int8_t* __restrict__ xq, int64_t ldq,
                                                         float* __restrict__ s_x,
                                                         int32_t* __restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= M) return;
  const int64_t nchunk = K >> 3;
  const uint16_t* row = x + t * ldx;
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * 64 + lane;
    v[c] = (j < nchunk) ? ld16(row + j * 8) : make_uint4(0, 0, 0, 0);
  }
  RowParams p;
  if (MODE == kDynSym || MODE == kDynAsym) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) minmax8(v[c], lo, hi);
    lo = wave_min(lo);
    hi = wave_max(hi);
    p = row_params<MODE>(lo, hi, s_in, zp_in);
    if (lane == 0) {
      s_x[t] = p.s;
      if (MODE == kDynAsym) zp[t] = p.zp;
    }
  } else {
    p = row_params<MODE>(0.0f, 0.0f, s_in, zp_in);
  }
  int8_t* orow = xq + t * ldq;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * 64 + lane;
    if (j < nchunk) *reinterpret_cast<uint2*>(orow + j * 8) = codes8<MODE>(v[c], p);
  }
}

// Any K: a first pass for the extremes, a second that re-reads and writes.
template <int MODE>
__global__ __launch_bounds__(256) void quant_rows_loop_kernel(const uint16_t* __restrict__ x,
                                                              int64_t M, int64_t K, int64_t ldx,
                                                              const float* __restrict__ s_in,
                                                              const int32_t* __restrict__ zp_in,
                                                              int8_t* __restrict__ xq, int64_t ldq,
                                                              float* __restrict__ s_x,
                                                              int32_t* __restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= M) return;
  const int64_t nchunk = K >> 3;
  const uint16_t* row = x + t * ldx;
  RowParams p;
  if (MODE == kDynSym || MODE == kDynAsym) {
    float lo = 0.0f, hi = 0.0f;
    for (int64_t j = lane; j < nchunk; j += 64) minmax8(ld16(row + j * 8), lo, hi);
    lo = wave_min(lo);
    hi = wave_max(hi);
    p = row_params<MODE>(lo, hi, s_in, zp_in);
    if (lane == 0) {
      s_x[t] = p.s;
      if (MODE == kDynAsym) zp[t] = p.zp;
    }
  } else {
    p = row_params<MODE>(0.0f, 0.0f, s_in, zp_in);
  }
  int8_t* orow = xq + t * ldq;
  for (int64_t j = lane; j < nchunk; j += 64)
    *reinterpret_cast<uint2*>(orow + j * 8) = codes8<MODE>(ld16(row + j * 8), p);
}

template <int MODE>
static hipError_t launch_mode(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const float* s_in, const int32_t* zp_in, int8_t* xq, int64_t ldq,
                              float* s_x, int32_t* zp, hipStream_t stream) {
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  const int64_t per_lane = (K / 8 + 63) / 64;  // 16-byte chunks per lane
#define W8A8_QLAUNCH(CHV)                                                                       \
  hipLaunchKernelGGL((quant_rows_kernel<MODE, CHV>), grid, block, 0, stream, x, M, K, ldx, s_in, \
                     zp_in, xq, ldq, s_x, zp)
  if (per_lane <= 1) W8A8_QLAUNCH(1);
  else if (per_lane <= 2) W8A8_QLAUNCH(2);
  else if (per_lane <= 4) W8A8_QLAUNCH(4);
  else if (per_lane <= 8) W8A8_QLAUNCH(8);
  else if (per_lane <= 16) W8A8_QLAUNCH(16);
  else if (per_lane <= 28) W8A8_QLAUNCH(28);
  else if (per_lane <= 32) W8A8_QLAUNCH(32);
  else
    hipLaunchKernelGGL((quant_rows_loop_kernel<MODE>), grid, block, 0, stream, x, M, K, ldx, s_in,
                       zp_in, xq, ldq, s_x, zp);
#undef W8A8_QLAUNCH
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int mode,
                               const float* s_in, const int32_t* zp_in, int8_t* xq, int64_t ldq,
                               float* s_x, int32_t* zp, hipStream_t stream) {
  switch (mode) {
    case kDynSym: return launch_mode<kDynSym>(x, M, K, ldx, s_in, zp_in, xq, ldq, s_x, zp, stream);
    case kDynAsym: return launch_mode<kDynAsym>(x, M, K, ldx, s_in, zp_in, xq, ldq, s_x, zp, stream);
    case kStaticSym:
      return launch_mode<kStaticSym>(x, M, K, ldx, s_in, zp_in, xq, ldq, s_x, zp, stream);
    default:
      return launch_mode<kStaticAsym>(x, M, K, ldx, s_in, zp_in, xq, ldq, s_x, zp, stream);
  }
}

}  // namespace w8a8
