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
// Layout: TPR threads own one row (TPR = 64, 256, 512 or 1024; several rows
// share a 256-thread workgroup when TPR = 64). The row is read once with 16-byte
// loads (8 bf16 per chunk, consecutive threads on consecutive chunks, so a
// wave instruction moves 1 KiB of contiguous HBM), held in registers (CH
// chunks per thread) while the extremes are reduced across lanes with DPP
// moves and across the row's waves through LDS, then written as 8-byte code
// stores. HBM traffic is the algorithmic 2 B read + 1 B written per element.
// Small batches use wide rows (more threads per row, fewer chunks per thread)
// to cut latency; large batches run several rounds of waves so that loading
// and computing overlap.
//
// Exactness: the absmax / min / max are exact, the scale is one IEEE binary32
// division, and each code is rint(fl(x / s)) with round-half-to-even, computed
// by the exact multiplication of rounding.h (the dynamic modes: one fused
// multiply-add gives the code with its zero point, a second one the distance
// to the nearest half-integer; about 6 VALU operations per element with the
// extremes; the true division only near a half-integer).

#include "device_common.h"
#include "launch.h"
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

template <int MODE, int TPR, int CH>
__global__ __launch_bounds__(TPR < 256 ? 256 : TPR) void quant_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ s_in, const int32_t* __restrict__ zp_in, int8_t* __restrict__ xq,
    int64_t ldq, float* __restrict__ s_x, int32_t* __restrict__ zp) {
  constexpr int BLOCK = TPR < 256 ? 256 : TPR;
  constexpr int RPB = BLOCK / TPR;           // rows per workgroup
  constexpr int WPR = TPR / 64;              // waves per row
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool row_ok = t < M;
  if (WPR == 1 && !row_ok) return;           // nothing below synchronises in that case
  const int64_t nchunk = K >> 3;
  const uint16_t* row = x + (row_ok ? t : 0) * ldx;
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    v[c] = (row_ok && j < nchunk) ? ld16(row + j * 8) : make_uint4(0, 0, 0, 0);
  }
  RowParams p;
  if (MODE == kDynSym || MODE == kDynAsym) {
    float lo = 0.0f, hi = 0.0f;
    if (MODE == kDynSym) {  // only the largest magnitude matters: hi = max |x|
#pragma unroll
      for (int c = 0; c < CH; ++c) absmax8(v[c], hi);
      hi = wave_extreme<true>(hi);
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) minmax8(v[c], lo, hi);
      lo = wave_extreme<false>(lo);
      hi = wave_extreme<true>(hi);
    }
    if (WPR > 1) {
      __shared__ float red_lo[RPB][WPR > 1 ? WPR : 1], red_hi[RPB][WPR > 1 ? WPR : 1];
      const int rb = threadIdx.x / TPR, wv = sub >> 6;
      if ((threadIdx.x & 63) == 0) {
        red_lo[rb][wv] = lo;
        red_hi[rb][wv] = hi;
      }
      __syncthreads();
      lo = red_lo[rb][0];
      hi = red_hi[rb][0];
#pragma unroll
      for (int i = 1; i < WPR; ++i) {
        lo = min_ieee(lo, red_lo[rb][i]);
        hi = max_ieee(hi, red_hi[rb][i]);
      }
    }
    if (!row_ok) return;
    p = row_params<MODE>(lo, hi, s_in, zp_in);
    if (sub == 0) {
      s_x[t] = p.s;
      if (MODE == kDynAsym) zp[t] = p.zp;
    }
  } else {
    if (!row_ok) return;
    p = row_params<MODE>(0.0f, 0.0f, s_in, zp_in);
  }
  int8_t* orow = xq + t * ldq;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    if (j < nchunk) *reinterpret_cast<uint2*>(orow + j * 8) = codes8<MODE>(v[c], p);
  }
}

template <int MODE, int TPR>
static void launch_tpr(int ch, dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M,
                       int64_t K, int64_t ldx, const float* s_in, const int32_t* zp_in, int8_t* xq,
                       int64_t ldq, float* s_x, int32_t* zp) {
  constexpr int BLOCK = TPR < 256 ? 256 : TPR;
#define W8A8_Q(CHV)                                                                           \
  hipLaunchKernelGGL((quant_kernel<MODE, TPR, CHV>), grid, dim3(BLOCK), 0, stream, x, M, K, ldx, \
                     s_in, zp_in, xq, ldq, s_x, zp)
  if (ch <= 1) W8A8_Q(1);
  else if (ch <= 2) W8A8_Q(2);
  else if (ch <= 4) W8A8_Q(4);
  else W8A8_Q(8);
#undef W8A8_Q
}

template <int MODE>
static hipError_t launch_mode(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const float* s_in, const int32_t* zp_in, int8_t* xq, int64_t ldq,
                              float* s_x, int32_t* zp, hipStream_t stream) {
  const int64_t nchunk = K / 8;
  // Threads per row: wide rows for small batches (latency). Large batches
  // also run 4 waves per row up to K = 16384: one wave per row leaves a
  // single round of waves on the chip at 8192 rows, which then load together
  // and compute together (8192 x 4096: 20 us at 4 waves per row against
  // 24 us at one, symmetric).
  // (Decode rows, input from HBM, M = 1..64: K = 4096 takes 2.2-2.9 us at 512
  // threads per row against 2.3-3.1 us at 256; K = 14336 is fastest at 1024.)
  int tpr;
  if (M <= 256)
    tpr = nchunk <= 64 ? 64 : (nchunk <= 256 ? 256 : (nchunk <= 512 ? 512 : 1024));
  else
    tpr = nchunk <= 128 ? 64 : (nchunk <= 2048 ? 256 : 1024);
  const int ch = (int)((nchunk + tpr - 1) / tpr);  // <= 8 since K <= 65536
  if (tpr == 64) {
    launch_tpr<MODE, 64>(ch, dim3((unsigned)((M + 3) / 4)), stream, x, M, K, ldx, s_in, zp_in, xq,
                         ldq, s_x, zp);
  } else if (tpr == 256) {
    launch_tpr<MODE, 256>(ch, dim3((unsigned)M), stream, x, M, K, ldx, s_in, zp_in, xq, ldq, s_x,
                          zp);
  } else if (tpr == 512) {
    launch_tpr<MODE, 512>(ch, dim3((unsigned)M), stream, x, M, K, ldx, s_in, zp_in, xq, ldq, s_x,
                          zp);
  } else {
    launch_tpr<MODE, 1024>(ch, dim3((unsigned)M), stream, x, M, K, ldx, s_in, zp_in, xq, ldq, s_x,
                           zp);
  }
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
