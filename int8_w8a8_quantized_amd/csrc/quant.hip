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

#include "launch.h"
#include "quant_common.h"

namespace w8a8 {

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

// ---------------------------------------------------------- FP8 activations
// E4M3 quantisation of the W8A8 FP8 scheme ("[SGLang] W4A8, W8A8, W4A4: 혼합
// 정밀도 양자화 스킴", 핵심 코드 분석 §1-§2): per token (s = absmax / 448),
// with a given per-tensor scale, or per token in groups of 128 along K (the
// block path's activation; scales stored group-major [G, M]). Each code is
// the true quotient x / s (one IEEE division), saturated at +-448 and
// rounded to the nearest E4M3 value, ties to even.
enum { kFp8Token = 0, kFp8Tensor = 1, kFp8Group = 2 };

// E4M3FN code of t, |t| <= 448 (not NaN). Below 2^-6 the values are the
// multiples of 2^-9 (codes 0..8, 8 being 2^-6 itself); above, the binary32
// mantissa is rounded to 3 bits (ties to even, a carry moves the exponent)
// and the exponent rebiased from 127 to 7. The sign bit is kept.
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  const uint32_t u = __float_as_uint(t);
  const float a = fabsf(t);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)rne(a * 512.0f);
  } else {
    uint32_t v = __float_as_uint(a);
    v += 0x7FFFFu + ((v >> 20) & 1u);
    mag = (((v >> 23) - 120u) << 3) | ((v >> 20) & 7u);
  }
  return ((u >> 24) & 0x80u) | mag;
}

// 8 bf16 values -> 8 E4M3 codes, x / s saturated at +-448.
__device__ __forceinline__ uint2 fp8_codes8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = e4m3_code(fminf(fmaxf(bf16_lo(w[i]) / s, -448.0f), 448.0f));
    c[2 * i + 1] = e4m3_code(fminf(fmaxf(bf16_hi(w[i]) / s, -448.0f), 448.0f));
  }
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// Largest magnitude over the 16 lanes of a DPP row (a group of 128 values
// spread 8 per lane), every lane of the row receiving it.
__device__ __forceinline__ float row16_max(float v) {
  auto op = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror
  v = op(v, dpp_move<0x140>(v));  // row_mirror
  return v;
}

// TPR threads own one row (TPR a multiple of 64, or 64 with 4 rows per
// workgroup); chunk j of 8 values is held by thread j % TPR in pass j / TPR,
// so the 16 chunks of a 128-group sit in one DPP row of 16 lanes.
template <int MODE, int TPR, int CH>
__global__ __launch_bounds__(TPR < 256 ? 256 : TPR) void quant_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, const float* __restrict__ s_in,
    uint8_t* __restrict__ xq, int64_t ldq, float* __restrict__ s_x) {
  constexpr int BLOCK = TPR < 256 ? 256 : TPR;
  constexpr int RPB = BLOCK / TPR, WPR = TPR / 64;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool row_ok = t < M;
  if (WPR == 1 && !row_ok) return;
  const int64_t nchunk = K >> 3;
  const uint16_t* row = x + (row_ok ? t : 0) * ldx;
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    v[c] = (row_ok && j < nchunk) ? ld16(row + j * 8) : make_uint4(0, 0, 0, 0);
  }
  float s_row = 1.0f;
  if (MODE == kFp8Token) {
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) absmax8(v[c], a);
    a = wave_extreme<true>(a);
    if (WPR > 1) {
      __shared__ float red[RPB][WPR > 1 ? WPR : 1];
      const int rb = threadIdx.x / TPR;
      if ((threadIdx.x & 63) == 0) red[rb][sub >> 6] = a;
      __syncthreads();
      a = red[rb][0];
#pragma unroll
      for (int i = 1; i < WPR; ++i) a = max_ieee(a, red[rb][i]);
    }
    if (!row_ok) return;
    s_row = a == 0.0f ? 1.0f : a / 448.0f;
    if (sub == 0) s_x[t] = s_row;
  } else if (MODE == kFp8Tensor) {
    if (!row_ok) return;
    s_row = *s_in;
  }
  if (!row_ok) return;
  uint8_t* orow = xq + t * ldq;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    float s = s_row;
    if (MODE == kFp8Group) {
      float a = 0.0f;
      absmax8(v[c], a);
      a = row16_max(a);  // chunks past K read as zeros
      s = a == 0.0f ? 1.0f : a / 448.0f;
      if ((sub & 15) == 0 && j < nchunk) s_x[(j >> 4) * M + t] = s;
    }
    if (j < nchunk) *reinterpret_cast<uint2*>(orow + j * 8) = fp8_codes8(v[c], s);
  }
}

hipError_t launch_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int mode,
                                   const float* s_in, uint8_t* xq, int64_t ldq, float* s_x, hipStream_t stream) {
  const int64_t nchunk = K / 8;
  int tpr;
  if (M <= 256)
    tpr = nchunk <= 64 ? 64 : (nchunk <= 256 ? 256 : 1024);
  else
    tpr = nchunk <= 128 ? 64 : (nchunk <= 2048 ? 256 : 1024);
  const int ch = (int)((nchunk + tpr - 1) / tpr);  // <= 8 since K <= 65536
#define W8A8_F8(MODEV, TPRV, CHV)                                                                         \
  hipLaunchKernelGGL((quant_fp8_kernel<MODEV, TPRV, CHV>),                                                \
                     dim3((unsigned)(TPRV < 256 ? (M + 3) / 4 : M)), dim3(TPRV < 256 ? 256 : TPRV), 0, stream, \
                     x, M, K, ldx, s_in, xq, ldq, s_x)
#define W8A8_F8_CH(MODEV, TPRV)                     \
  do {                                              \
    if (ch <= 1) W8A8_F8(MODEV, TPRV, 1);           \
    else if (ch <= 2) W8A8_F8(MODEV, TPRV, 2);      \
    else if (ch <= 4) W8A8_F8(MODEV, TPRV, 4);      \
    else W8A8_F8(MODEV, TPRV, 8);                   \
  } while (0)
#define W8A8_F8_TPR(MODEV)                                                    \
  do {                                                                        \
    if (tpr == 64) W8A8_F8_CH(MODEV, 64);                                     \
    else if (tpr == 256) W8A8_F8_CH(MODEV, 256);                              \
    else W8A8_F8_CH(MODEV, 1024);                                             \
  } while (0)
  if (mode == kFp8Token) W8A8_F8_TPR(kFp8Token);
  else if (mode == kFp8Tensor) W8A8_F8_TPR(kFp8Tensor);
  else W8A8_F8_TPR(kFp8Group);
#undef W8A8_F8_TPR
#undef W8A8_F8_CH
#undef W8A8_F8
  return hipGetLastError();
}

// ---------------------------------------------- RMS normalisation + codes
// The quantiser fused into the op before it in a decoder layer: the RMS
// normalisation of the bf16 rows (after the optional residual add) and the
// per-token symmetric quantisation of its bf16 output, in one pass over the
// row held in registers. Rounding, per element: h = bf16(x + residual)
// (binary32 carries more than twice bf16's 8 significant bits, so rounding
// the binary32 sum of two bf16 values to bf16 gives the correctly rounded
// sum: a double rounding through that width is innocuous); y = bf16(h * gamma / sqrt(mean(h^2) + eps)) with the mean
// square, its root and the products in binary64 (every h^2 and h * gamma is
// exact there), so y is the correctly rounded value except within about
// 2^-45 of a bf16 rounding boundary (a binary32 evaluation with a binary64
// fallback near those boundaries measured slower: the fallback code doubled
// the kernel and its registers); the codes and the scale are the quantiser's own
// (codes8 on y). HBM traffic per element: 2 B in (+2 B residual in and out),
// 1 B out (+2 B for y when it is asked for); gamma comes from the caches.

// binary64 -> bf16, round to nearest even: rounding to binary32 toward zero
// with a sticky bit for any inexactness (round to odd) keeps the second
// rounding, binary32 -> bf16, correct.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double d) {
  const float f = (float)d;
  const double back = (double)f;
  uint32_t u = __float_as_uint(f);
  if (back != d && d == d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // rounded away from zero: one binary32 step back toward it
    u |= 1u;
  }
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int TPR>
__device__ __forceinline__ double row_sum_f64(double v, double* red) {
  constexpr int WPR = TPR / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (WPR > 1) {
    const int rb = (threadIdx.x / TPR), wv = (threadIdx.x % TPR) >> 6;
    if ((threadIdx.x & 63) == 0) red[rb * WPR + wv] = v;
    __syncthreads();
    v = red[rb * WPR];
#pragma unroll
    for (int i = 1; i < WPR; ++i) v += red[rb * WPR + i];
  }
  return v;
}

template <int TPR, int CH>
__global__ __launch_bounds__(TPR < 256 ? 256 : TPR) void rmsnorm_quant_kernel(
    const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint16_t* res, int64_t ldr, uint16_t* y, int64_t ldy, int8_t* __restrict__ xq, int64_t ldq,
    float* __restrict__ s_x) {
  // x, res and y may be one buffer (the residual and the normalised rows may
  // overwrite x): each element is read and written by the same thread, all
  // reads first, so no qualifier promises them apart
  constexpr int BLOCK = TPR < 256 ? 256 : TPR;
  constexpr int RPB = BLOCK / TPR;  // rows per workgroup
  constexpr int WPR = TPR / 64;     // waves per row
  __shared__ double red_d[RPB * WPR];
  __shared__ float red_f[RPB * WPR];
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool row_ok = t < M;
  if (WPR == 1 && !row_ok) return;  // nothing below synchronises in that case
  const int64_t nchunk = K >> 3;
  const int64_t tr = row_ok ? t : 0;
  // every load goes out first (x, the residual, gamma): one round trip
  uint4 v[CH], rv[CH], gv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    const bool in = row_ok && j < nchunk;
    v[c] = in ? ld16(x + tr * ldx + j * 8) : make_uint4(0, 0, 0, 0);
    rv[c] = (in && res != nullptr) ? ld16(res + tr * ldr + j * 8) : make_uint4(0, 0, 0, 0);
    gv[c] = j < nchunk ? ld16(gamma + j * 8) : make_uint4(0, 0, 0, 0);
  }
  if (res != nullptr) {  // h = bf16(x + residual), which becomes the residual
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t j = (int64_t)c * TPR + sub;
      if (!(row_ok && j < nchunk)) continue;
      const uint4 r = rv[c];
      const uint32_t a[4] = {v[c].x, v[c].y, v[c].z, v[c].w}, b[4] = {r.x, r.y, r.z, r.w};
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[i] = pack_bf16x2(bf16_lo(a[i]) + bf16_lo(b[i]), bf16_hi(a[i]) + bf16_hi(b[i]));
      v[c] = make_uint4(h[0], h[1], h[2], h[3]);
      st16(res + tr * ldr + j * 8, v[c]);
    }
  }
  // mean square in binary64
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double lo = (double)bf16_lo(w[i]), hi = (double)bf16_hi(w[i]);
      ss = __builtin_fma(lo, lo, ss);
      ss = __builtin_fma(hi, hi, ss);
    }
  }
  ss = row_sum_f64<TPR>(ss, red_d);
  const double inv = 1.0 / __builtin_sqrt(ss / (double)K + (double)eps);
  // y = bf16(h * gamma * inv) in binary64 and its absmax
  auto norm = [&](float hv, float gvv) __attribute__((always_inline)) -> uint32_t {
    return f64_to_bf16_bits((double)hv * (double)gvv * inv);
  };
  float am = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w}, g[4] = {gv[c].x, gv[c].y, gv[c].z, gv[c].w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = norm(bf16_lo(w[i]), bf16_lo(g[i])) | (norm(bf16_hi(w[i]), bf16_hi(g[i])) << 16);
    v[c] = make_uint4(o[0], o[1], o[2], o[3]);
    absmax8(v[c], am);
  }
  am = wave_extreme<true>(am);
  if (WPR > 1) {
    const int rb = threadIdx.x / TPR, wv = sub >> 6;
    if ((threadIdx.x & 63) == 0) red_f[rb * WPR + wv] = am;
    __syncthreads();
    am = red_f[rb * WPR];
#pragma unroll
    for (int i = 1; i < WPR; ++i) am = max_ieee(am, red_f[rb * WPR + i]);
  }
  if (!row_ok) return;
  const RowParams p = row_params<kDynSym>(0.0f, am, nullptr, nullptr);
  if (sub == 0) s_x[t] = p.s;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    if (j >= nchunk) continue;
    *reinterpret_cast<uint2*>(xq + t * ldq + j * 8) = codes8<kDynSym>(v[c], p);
    if (y != nullptr) st16(y + t * ldy + j * 8, v[c]);
  }
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                float eps, uint16_t* residual, int64_t ldr, uint16_t* y, int64_t ldy, int8_t* xq,
                                int64_t ldq, float* s_x, hipStream_t stream) {
  // the quantiser's threads-per-row table (wide rows for small batches)
  const int64_t nchunk = K / 8;
  int tpr;
  if (M <= 256)
    tpr = nchunk <= 64 ? 64 : (nchunk <= 256 ? 256 : (nchunk <= 512 ? 512 : 1024));
  else
    tpr = nchunk <= 128 ? 64 : (nchunk <= 2048 ? 256 : 1024);
  const int ch = (int)((nchunk + tpr - 1) / tpr);  // <= 8 since K <= 65536
#define W8A8_RN(TPRV, CHV)                                                                                   \
  hipLaunchKernelGGL((rmsnorm_quant_kernel<TPRV, CHV>), dim3((unsigned)(TPRV < 256 ? (M + 3) / 4 : M)),       \
                     dim3(TPRV < 256 ? 256 : TPRV), 0, stream, x, M, K, ldx, gamma, eps, residual, ldr, y, ldy, \
                     xq, ldq, s_x)
#define W8A8_RN_CH(TPRV)                          \
  do {                                            \
    if (ch <= 1) W8A8_RN(TPRV, 1);                \
    else if (ch <= 2) W8A8_RN(TPRV, 2);           \
    else if (ch <= 4) W8A8_RN(TPRV, 4);           \
    else W8A8_RN(TPRV, 8);                        \
  } while (0)
  if (tpr == 64) W8A8_RN_CH(64);
  else if (tpr == 256) W8A8_RN_CH(256);
  else if (tpr == 512) W8A8_RN_CH(512);
  else W8A8_RN_CH(1024);
#undef W8A8_RN_CH
#undef W8A8_RN
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
