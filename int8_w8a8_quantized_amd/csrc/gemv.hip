// Decode-shaped (M <= 64) int8 GEMM: a weight-streaming kernel.
//
// Same product and fused epilogue as the prefill GEMM ("[SGLang] W4A8, W8A8,
// W4A4: 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3-§4), but with a handful of
// token rows the work is bound by reading the N x K int8 weight from HBM once.
//
// A workgroup owns 16 weight rows (one MFMA column block) over the whole K.
// Its waves split K in interleaved 64-byte steps, so at any moment the
// workgroup reads a contiguous stretch of every one of its 16 rows. Each lane
// loads the 16 bytes it feeds to v_mfma_i32_16x16x64_i8 straight from HBM
// into registers (no LDS staging: each weight byte is used exactly once), U
// steps ahead to keep enough bytes in flight; the token rows (M padded to
// 16-row MFMA blocks, MF of them) come from L2, where the small activation
// matrix stays resident. The waves' int32 partial sums are added in LDS and
// the first wave applies the epilogue. Integer sums are exact in any order.

#include "gemm_common.h"

namespace w8a8 {

template <int MF, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void gemv_i8_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int frag_row = lane & 15, kgrp = (lane >> 4) * 16;
  const int64_t n = (int64_t)blockIdx.x * 16 + frag_row;
  const bool n_ok = n < a.N;
  const int8_t* bp = a.B + (n_ok ? n : 0) * a.ldb + kgrp;
  const int8_t* ap[MF];
  bool a_ok[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int64_t m = f * 16 + frag_row;
    a_ok[f] = m < a.M;
    ap[f] = a.A + (a_ok[f] ? m : 0) * a.lda + kgrp;
  }
  i32x4 acc[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) acc[f] = i32x4{0, 0, 0, 0};

  const int64_t nsteps = (a.K + 63) / 64;
  for (int64_t s = wave; s < nsteps; s += (int64_t)WAVES * U) {
    uint4 b[U], x[U][MF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = s + (int64_t)u * WAVES;
      const int64_t k = ks * 64;
      const bool k_ok = ks < nsteps && k + kgrp < a.K;
      b[u] = (k_ok && n_ok) ? ld16(bp + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < MF; ++f)
        x[u][f] = (k_ok && a_ok[f]) ? ld16(ap[f] + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < MF; ++f) acc[f] = mfma16x16x64(as_i32x4(x[u][f]), as_i32x4(b[u]), acc[f]);
  }

  __shared__ i32x4 red[WAVES][MF][64];
  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < MF; ++f) red[wave][f][lane] = acc[f];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < WAVES; ++w)
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[f] += red[w][f][lane];

  const EpiCol col = load_col(a, n, a.s_w, a.bias);
#pragma unroll
  for (int f = 0; f < MF; ++f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = f * 16 + (lane >> 4) * 4 + r;
      EpiRow er;
      er.ok = m < a.M;
      er.out_row = m;
      const int64_t mm = er.ok ? m : 0;
      er.sx = a.sx_per_token ? a.s_x[mm] : a.s_x[0];
      er.zp = (a.azp_mode == 1) ? a.zp[mm] : 0;
      epilogue_store(a, er, col, n, acc[f][r]);
    }
  }
}

hipError_t launch_decode_mm(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 15) / 16));
  constexpr int W = 8, U = 4;
  const dim3 block(W * 64);
  if (a.M <= 16)
    hipLaunchKernelGGL((gemv_i8_kernel<1, W, U>), grid, block, 0, stream, a);
  else if (a.M <= 32)
    hipLaunchKernelGGL((gemv_i8_kernel<2, W, U>), grid, block, 0, stream, a);
  else if (a.M <= 48)
    hipLaunchKernelGGL((gemv_i8_kernel<3, W, U>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemv_i8_kernel<4, W, U>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace w8a8
