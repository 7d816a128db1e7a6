// Decode-shaped (M <= 64) int8 GEMM: a weight-streaming kernel.
//
// Same product and fused epilogue as the prefill GEMM ("[SGLang] W4A8, W8A8,
// W4A4: 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3-§4), but with a handful of
// token rows the time is reading the N x K int8 weight from HBM once.
//
// Work unit: a 64-row slice of the weight (4 MFMA column blocks) times a
// contiguous range of K ("split"). A workgroup of 4 waves takes one unit; its
// waves interleave over the range in 64-byte steps, so at any moment the
// workgroup reads a contiguous stretch of each of its 64 rows. Every lane
// loads the 16 bytes it feeds to v_mfma_i32_16x16x64_i8 straight from HBM
// into registers (non-temporal: each weight byte is used once), U steps ahead
// so that ~32 KiB per workgroup are in flight. The token rows (M padded to
// 16-row MFMA blocks) come from L2; each weight fragment is reused for all M
// rows and each activation fragment for all 64 weight rows, so activation
// traffic from L2 equals M/64 of the weight traffic.
//
// Reduction: the waves' int32 partial tiles are added in LDS. With one split
// the workgroup applies the epilogue directly. With several, each workgroup
// adds its tile into an int32 workspace with device-scope atomics; the last
// one to arrive (a per-slice arrival counter) takes the sums out with atomic
// exchanges (leaving zeros), applies the epilogue and resets the counter, so
// the next call finds the workspace clean. Integer sums are exact in any
// order, so the result does not depend on the arrival order.

#include <algorithm>

#include "gemm_common.h"

namespace w8a8 {

namespace {
constexpr int kNF = 4;             // 16-row weight blocks per unit
constexpr int kTN = kNF * 16;      // weight rows per unit
constexpr int kWaves = 4;
}  // namespace

__device__ __forceinline__ void epilogue_one(const GemmArgs& a, int64_t m, int64_t n, int acc) {
  EpiRow er;
  er.ok = true;
  er.out_row = m;
  er.sx = a.sx_per_token ? a.s_x[m] : a.s_x[0];
  er.zp = (a.azp_mode == 1) ? a.zp[m] : 0;
  const EpiCol col = load_col(a, n, a.s_w, a.bias);
  epilogue_store(a, er, col, n, acc);
}

template <int MF, int U>
__global__ __launch_bounds__(kWaves * 64) void gemv_i8_kernel(GemmArgs a, int splits,
                                                              int64_t steps_per_split,
                                                              int32_t* __restrict__ ws,
                                                              int32_t* __restrict__ arrivals) {
  constexpr int TM = MF * 16;
  constexpr int NT = kWaves * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int frag_row = lane & 15, kgrp = (lane >> 4) * 16;
  const int64_t tile = blockIdx.x / splits;
  const int split = (int)(blockIdx.x - tile * splits);
  const int64_t n0 = tile * kTN;
  const int64_t nsteps = (a.K + 63) / 64;
  const int64_t s_begin = (int64_t)split * steps_per_split;
  const int64_t s_end = min(nsteps, s_begin + steps_per_split);

  const int8_t* bp[kNF];
  bool b_ok[kNF];
#pragma unroll
  for (int j = 0; j < kNF; ++j) {
    const int64_t n = n0 + j * 16 + frag_row;
    b_ok[j] = n < a.N;
    bp[j] = a.B + (b_ok[j] ? n : 0) * a.ldb + kgrp;
  }
  const int8_t* ap[MF];
  bool a_ok[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int64_t m = f * 16 + frag_row;
    a_ok[f] = m < a.M;
    ap[f] = a.A + (a_ok[f] ? m : 0) * a.lda + kgrp;
  }
  i32x4 acc[MF][kNF];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[f][j] = i32x4{0, 0, 0, 0};

  for (int64_t s = s_begin + wave; s < s_end; s += (int64_t)kWaves * U) {
    uint4 b[U][kNF], x[U][MF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ks = s + (int64_t)u * kWaves;
      const int64_t k = ks * 64;
      const bool k_ok = ks < s_end && k + kgrp < a.K;
#pragma unroll
      for (int j = 0; j < kNF; ++j)
        b[u][j] = (k_ok && b_ok[j]) ? ldnt16(bp[j] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < MF; ++f)
        x[u][f] = (k_ok && a_ok[f]) ? ld16(ap[f] + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int j = 0; j < kNF; ++j)
          acc[f][j] = mfma16x16x64(as_i32x4(x[u][f]), as_i32x4(b[u][j]), acc[f][j]);
  }

  // ---- add the waves' partial tiles (row-major TM x 64 int32 per wave)
  __shared__ int32_t part[kWaves][TM * kTN];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < kNF; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[wave][(f * 16 + (lane >> 4) * 4 + r) * kTN + j * 16 + frag_row] = acc[f][j][r];
  __syncthreads();

  const int rows = (int)min<int64_t>(a.M, TM);
  if (splits == 1) {
    for (int e = tid; e < rows * kTN; e += NT) {
      const int m = e / kTN, c = e % kTN;
      const int64_t n = n0 + c;
      if (n >= a.N) continue;
      int v = part[0][e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += part[w][e];
      epilogue_one(a, m, n, v);
    }
    return;
  }

  // Every value this workgroup hands to another one moves through device-scope
  // atomic read-modify-writes, which are performed at the device's point of
  // coherence. So no cache-wide fence is needed (on this multi-XCD part a
  // device-scope fence writes back and invalidates the whole L2): it is
  // enough that each thread's adds have completed (vmcnt drained) before the
  // workgroup announces its arrival, and that the last arriver reads the sums
  // with atomic exchanges, which also return the workspace to zero.
  for (int e = tid; e < rows * kTN; e += NT) {
    const int m = e / kTN, c = e % kTN;
    const int64_t n = n0 + c;
    if (n >= a.N) continue;
    int v = part[0][e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += part[w][e];
    atomicAdd(ws + m * a.N + n, v);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = (atomicAdd(arrivals + tile, 1) == splits - 1);
  __syncthreads();
  if (!last) return;
  for (int e = tid; e < rows * kTN; e += NT) {
    const int m = e / kTN, c = e % kTN;
    const int64_t n = n0 + c;
    if (n >= a.N) continue;
    epilogue_one(a, m, n, atomicExch(ws + m * a.N + n, 0));
  }
  if (tid == 0) atomicExch(arrivals + tile, 0);
}

// Workspace of the split path: int32 sums [M, N], then one arrival counter per
// 64-row slice, rounded up to 256 bytes.
size_t decode_workspace_bytes(int64_t M, int64_t N) {
  const int64_t tiles = (N + kTN - 1) / kTN;
  const size_t b = (size_t)(M * N + tiles) * sizeof(int32_t);
  return (b + 255) & ~size_t(255);
}

const char* decode_kernel_name(int64_t M) {
  if (M <= 16) return "gemv_i8_kernel<1, 4>";
  if (M <= 32) return "gemv_i8_kernel<2, 4>";
  if (M <= 48) return "gemv_i8_kernel<3, 2>";
  return "gemv_i8_kernel<4, 2>";
}

hipError_t launch_decode_mm(const GemmArgs& a, void* workspace, size_t ws_bytes, int num_cus,
                            hipStream_t stream) {
  const int64_t tiles = (a.N + kTN - 1) / kTN;
  const int64_t nsteps = (a.K + 63) / 64;
  // Aim for two workgroups per compute unit; never give a wave an empty range.
  const int64_t target = 2 * (int64_t)num_cus;
  int64_t splits = (target + tiles / 2) / tiles;
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, nsteps / kWaves));
  if (splits > 1 && (workspace == nullptr || ws_bytes < decode_workspace_bytes(a.M, a.N))) splits = 1;
  int64_t sps = (nsteps + splits - 1) / splits;
  splits = (nsteps + sps - 1) / sps;
  int32_t* ws = static_cast<int32_t*>(workspace);
  int32_t* arrivals = ws ? ws + a.M * a.N : nullptr;
  const dim3 grid((unsigned)(tiles * splits)), block(kWaves * 64);
#define W8A8_GEMV(MFV, UV)                                                                  \
  hipLaunchKernelGGL((gemv_i8_kernel<MFV, UV>), grid, block, 0, stream, a, (int)splits, sps, \
                     ws, arrivals)
  if (a.M <= 16) W8A8_GEMV(1, 4);
  else if (a.M <= 32) W8A8_GEMV(2, 4);
  else if (a.M <= 48) W8A8_GEMV(3, 2);
  else W8A8_GEMV(4, 2);
#undef W8A8_GEMV
  return hipGetLastError();
}

}  // namespace w8a8
