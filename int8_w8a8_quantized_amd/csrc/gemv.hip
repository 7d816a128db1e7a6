// Decode-shaped (M <= 64) int8 GEMM: weight-streaming kernels.
//
// Same product and fused epilogue as the prefill GEMM ("[SGLang] W4A8, W8A8,
// W4A4: 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3-§4), but with a handful of
// token rows the time is reading the N x K int8 weight from HBM once, so the
// kernels are built around the HBM access pattern and the bytes in flight.
//
// Main kernel (K a multiple of 128), gemv_dma_kernel: a workgroup of 4
// waves owns 64 weight rows and a contiguous range of K (one of `splits`
// ranges). Weights and the (M padded to 16-row MFMA blocks) activations
// travel HBM/L2 -> LDS with the direct-to-LDS load, one wave instruction
// moving 8 rows x 128 bytes -- whole cache lines per row, the pattern that
// streams HBM at full rate (MFMA operand order, 16 rows x 64 bytes per
// instruction, reaches only about 60-70% of it) -- into a ring of NS stages
// of 128 bytes of K, so NS - 1 stages are in flight per workgroup. Chunks are
// XOR-swizzled within a row as in the prefill GEMM, so each wave's fragment
// reads (16 rows x one 16-byte chunk) hit distinct banks. Wave w multiplies
// weight rows 16w..16w+15 with all activation blocks with
// v_mfma_i32_16x16x64_i8. With one range the workgroup applies the epilogue
// from registers; with several, each workgroup stores its int32 partial tile
// to a caller workspace and the last one to arrive for the row block (an
// arrival counter) adds the partials, applies the epilogue and resets the
// counter (partials and counter through agent-scope
// atomics, no cache-wide fences). Integer sums are exact in any order.
//
// General kernel (any K that is a multiple of 16), gemv_i8_kernel: operands
// go straight from memory into MFMA registers, as described above it.

#include <algorithm>

#include "gemm_common.h"

namespace w8a8 {

typedef __attribute__((address_space(3))) void* lds_void_ptr_g;
typedef __attribute__((address_space(1))) void* global_void_ptr_g;

template <int N>
__device__ __forceinline__ void gemv_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void gemv_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// Chunk position of logical 16-byte chunk c of an 8-chunk (128-byte) row r:
// distinct banks for 16-byte reads of 8 (32-bank view) or 16 (64-bank view)
// consecutive rows at one chunk.
__device__ __forceinline__ int gemv_swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

template <int MF, int NS>
__global__ __launch_bounds__(256) void gemv_dma_kernel(GemmArgs a, int splits, int steps_per_split,
                                                       int32_t* __restrict__ part,
                                                       int32_t* __restrict__ counters) {
  constexpr int BN = 64, BK = 128;
  constexpr int XR = MF * 16;                    // activation rows held in LDS
  constexpr int STAGE = (BN + XR) * BK;
  constexpr int NI = (BN + XR) / 8;              // 1-KiB load instructions per stage
  constexpr int Q = (NI + 3) / 4;                // per wave (the last ones may repeat)
  static_assert((NS - 2) * Q <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int64_t n0 = (int64_t)rb * BN;
  const int nsteps = (int)(a.K / BK);
  const int s_begin = sp * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);
  const int nk = max(s_end - s_begin, 0);

  // ---- DMA sources: instruction j (this wave's q-th) fills tile rows
  // 8j..8j+7 (weights for j < BN/8, activations after); lane l writes row
  // +l/8, physical chunk l%8, which holds logical chunk (l%8) ^ swz(row).
  const int8_t* src[Q];
  int dst[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = min(wave * Q + q, NI - 1);
    const int trow = 8 * j + (lane >> 3);        // row within the stage
    const int lch = (lane & 7) ^ gemv_swz(trow);
    if (trow < BN) {
      src[q] = a.B + min(n0 + trow, a.N - 1) * a.ldb + lch * 16;
    } else {
      const int64_t m = min<int64_t>(trow - BN, a.M - 1);  // rows past M repeat the last one
      src[q] = a.A + m * a.lda + lch * 16;
    }
    dst[q] = j * 1024;
  }
  auto issue = [&](int kt_src, int kt_dst) __attribute__((always_inline)) {
    int8_t* st = smem + (kt_dst % NS) * STAGE;
    const int64_t k0 = (int64_t)(s_begin + kt_src) * BK;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      __builtin_amdgcn_global_load_lds((global_void_ptr_g)(src[q] + k0), (lds_void_ptr_g)(st + dst[q]),
                                       16, 0, 0);
  };

  // ---- fragments: wave w reads weight rows 16w + lane%16, activation rows
  // 16f + lane%16, logical chunk 4*ks + lane/16
  const int fr = lane & 15;
  const int w_off = (16 * wave + fr) * BK;
  const int w_sw = gemv_swz(16 * wave + fr);
  i32x4 acc[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) acc[f] = i32x4{0, 0, 0, 0};

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(min(s, nk - 1), s);
  }
  for (int kt = 0; kt < nk; ++kt) {
    gemv_wait_vmcnt<(NS - 2) * Q>();
    gemv_barrier();  // stage kt has landed everywhere; stage kt-1 is retired
    issue(min(kt + NS - 1, nk - 1), kt + NS - 1);  // past the end: a harmless reload
    const int8_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 4 * ks + (lane >> 4);
      const i32x4 wf = *reinterpret_cast<const i32x4*>(st + w_off + ((c ^ w_sw) * 16));
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        const int xr = BN + 16 * f + fr;
        const i32x4 xf = *reinterpret_cast<const i32x4*>(st + xr * BK + ((c ^ gemv_swz(xr)) * 16));
        acc[f] = mfma16x16x64(xf, wf, acc[f]);
      }
    }
  }
  gemv_wait_vmcnt<0>();  // the trailing reloads land before the workgroup ends

  // ---- results: lane holds rows 16f + 4*(lane/16) + r of column n0 + 16w + lane%16
  const int64_t n = n0 + 16 * wave + fr;
  if (splits == 1) {
    const EpiCol col = load_col(a, n, a.s_w, a.bias);
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 16 * f + 4 * (lane >> 4) + r;
        if (m >= a.M) continue;
        EpiRow er;
        er.ok = true;
        er.out_row = m;
        er.sx = a.sx_per_token ? a.s_x[m] : a.s_x[0];
        er.zp = (a.azp_mode == 1) ? a.zp[m] : 0;
        epilogue_store(a, er, col, n, acc[f][r]);
      }
    return;
  }

  // split K: partial tiles [splits][M][N], then the last arriver sums them.
  // Partials are written and read with agent-scope atomic stores / loads,
  // which go to and come from the device's point of coherence (past the
  // per-XCD L2s), so neither side needs a cache-wide fence (on this part a
  // release fence writes back the whole L2, which costs more than the
  // kernel): each thread's stores have completed (vmcnt drained, then the
  // barrier) before the workgroup takes its arrival number, and the last
  // arriver's loads are issued after it has seen the count.
  if (n < a.N) {
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 16 * f + 4 * (lane >> 4) + r;
        if (m < a.M)
          __hip_atomic_store(part + ((int64_t)sp * a.M + m) * a.N + n, acc[f][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  gemv_wait_vmcnt<0>();
  __syncthreads();
  int& last = *reinterpret_cast<int*>(smem);  // the stage ring is idle by now
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(counters + rb, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last = prev == splits - 1;
    // the last arriver leaves the counter at zero for the next call
    if (last) __hip_atomic_store(counters + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const int rows = (int)min<int64_t>(a.M, XR);
  for (int e = tid; e < rows * BN; e += 256) {
    const int m = e / BN;
    const int64_t nn = n0 + e % BN;
    if (nn >= a.N) continue;
    int v = 0;
    for (int s2 = 0; s2 < splits; ++s2)
      v += __hip_atomic_load(part + ((int64_t)s2 * a.M + m) * a.N + nn, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    EpiRow er;
    er.ok = true;
    er.out_row = m;
    er.sx = a.sx_per_token ? a.s_x[m] : a.s_x[0];
    er.zp = (a.azp_mode == 1) ? a.zp[m] : 0;
    const EpiCol col = load_col(a, nn, a.s_w, a.bias);
    epilogue_store(a, er, col, nn, v);
  }
}

// ------------------------------------------------------------- general kernel
// A workgroup of W waves owns 16 * NB weight rows over the whole K (no
// cross-workgroup reduction). K is cut into 64-byte steps (one
// v_mfma_i32_16x16x64_i8 per 16 x 16 block), dealt to the waves in chunks of
// U consecutive steps; each wave keeps a ring of U steps of loads in flight,
// every lane loading the 16 bytes it feeds to the MFMA straight into
// registers. Loads are branch-free: a step past the end of the wave's range
// reloads a valid address and is not used; activation chunks past K or M are
// zeros. The waves' partial tiles meet in LDS through integer atomic adds.
template <int MF, int NB, int W, int U>
__global__ __launch_bounds__(W * 64) void gemv_i8_kernel(GemmArgs a) {
  constexpr int TN = NB * 16, TM = MF * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int frag_row = lane & 15, kgrp = (lane >> 4) * 16;
  const int64_t n0 = (int64_t)blockIdx.x * TN;

  __shared__ int32_t sums[TM * TN];
  for (int e = tid; e < TM * TN; e += W * 64) sums[e] = 0;

  // weight rows of this lane (clamped: rows past N load row N-1, never stored)
  const int8_t* bp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    bp[j] = a.B + min(n0 + j * 16 + frag_row, a.N - 1) * a.ldb + kgrp;
  // activation rows of this lane (rows past M are zeros)
  const int8_t* ap[MF];
  bool a_ok[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int64_t m = f * 16 + frag_row;
    a_ok[f] = m < a.M;
    ap[f] = a.A + (a_ok[f] ? m : 0) * a.lda + kgrp;
  }

  const int nsteps = (int)((a.K + 63) / 64);
  const int nchunks = (nsteps + U - 1) / U;
  i32x4 acc[MF][NB];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[f][j] = i32x4{0, 0, 0, 0};

  u32x4 wb[U][NB], xb[U][MF];
  const u32x4 z = {0u, 0u, 0u, 0u};
  // Load step `step` into ring slot u; a step past the end reloads step 0.
  auto load_step = [&](int u, int step) __attribute__((always_inline)) {
    const bool live = step < nsteps;
    const int64_t k = (int64_t)(live ? step : 0) * 64;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      wb[u][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[j] + k));
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const bool ok = a_ok[f] && live && k + kgrp < a.K;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ap[f] + (ok ? k : 0));
      xb[u][f] = ok ? v : z;
    }
  };
  auto compute = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[f][j] = mfma16x16x64(__builtin_bit_cast(i32x4, xb[u][f]),
                                 __builtin_bit_cast(i32x4, wb[u][j]), acc[f][j]);
  };

  // chunks wave, wave + W, wave + 2W, ...; the next chunk's loads go out as
  // the current chunk's steps are consumed
  int c = wave;
  if (c < nchunks) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(u, c * U + u);
    for (; c < nchunks; c += W) {
      const int next = c + W;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int step = c * U + u;
        // a step of the last chunk past nsteps holds a reload of step 0: skip it
        if (step < nsteps) compute(u);
        load_step(u, next < nchunks ? next * U + u : nsteps);
      }
    }
  }

  // ---- add the waves' partial tiles in LDS: lane holds rows
  // 4*(lane/16)..+3 of column lane%16 of each 16x16 block
  __syncthreads();
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = f * 16 + (lane >> 4) * 4 + r;
        if (m < a.M) atomicAdd(&sums[m * TN + j * 16 + frag_row], acc[f][j][r]);
      }
  __syncthreads();

  const int rows = (int)min<int64_t>(a.M, TM);
  for (int e = tid; e < rows * TN; e += W * 64) {
    const int m = e / TN, cn = e % TN;
    const int64_t n = n0 + cn;
    if (n >= a.N) continue;
    EpiRow er;
    er.ok = true;
    er.out_row = m;
    er.sx = a.sx_per_token ? a.s_x[m] : a.s_x[0];
    er.zp = (a.azp_mode == 1) ? a.zp[m] : 0;
    const EpiCol col = load_col(a, n, a.s_w, a.bias);
    epilogue_store(a, er, col, n, sums[e]);
  }
}

namespace {

constexpr int kGemvRows = 64;  // weight rows per workgroup of the main kernel
constexpr int kCounters = 4096;  // arrival counters at the head of the workspace

// Launch shape of the main kernel: LDS stages and K ranges per row block,
// from a sweep over the Llama-3-8B decode linears (M in {1, 8, 32, 64},
// K x N in {4096 x 6144, 4096 x 4096, 4096 x 28672, 14336 x 4096}):
//  - many row blocks (N >= 16384): enough workgroups already; M <= 16 still
//    gains from two K ranges;
//  - long K (>= 8192) with few row blocks: four K ranges;
//  - otherwise one range (two for M <= 16).
// Larger M pays for every extra range with M x N int32 of partial sums.
struct GemvCfg {
  int ns, splits;
};

int gemv_mf(int64_t M) { return (int)std::min<int64_t>((M + 15) / 16, 4); }

GemvCfg gemv_cfg(int64_t M, int64_t N, int64_t K) {
  const int mf = gemv_mf(M);
  const int64_t blocks = (N + kGemvRows - 1) / kGemvRows;
  const int64_t nsteps = K / 128;
  GemvCfg c;
  if (mf == 1) c = blocks >= 256 ? GemvCfg{4, 2} : (nsteps >= 64 ? GemvCfg{4, 4} : GemvCfg{8, 2});
  else if (mf == 2) c = blocks >= 256 ? GemvCfg{6, 1} : (nsteps >= 64 ? GemvCfg{6, 4} : GemvCfg{4, 1});
  else c = blocks >= 256 ? GemvCfg{5, 1} : (nsteps >= 64 ? GemvCfg{5, 4} : GemvCfg{5, 1});
  if (K % 128 != 0 || blocks > kCounters) c.splits = 1;
  c.splits = (int)std::max<int64_t>(1, std::min<int64_t>(c.splits, nsteps));
  return c;
}

int gemv_splits(int64_t M, int64_t N, int64_t K) { return gemv_cfg(M, N, K).splits; }

template <int MF, int NS>
hipError_t launch_dma(const GemmArgs& a, int splits, int32_t* part, int32_t* counters,
                      hipStream_t stream) {
  static_assert((kGemvRows + MF * 16) * 128 * NS <= 80 * 1024, "two workgroups per CU");
  const int64_t nsteps = a.K / 128;
  const int sps = (int)((nsteps + splits - 1) / splits);
  const int64_t blocks = (a.N + kGemvRows - 1) / kGemvRows;
  hipLaunchKernelGGL((gemv_dma_kernel<MF, NS>), dim3((unsigned)(blocks * splits)), dim3(256), 0,
                     stream, a, splits, sps, part, counters);
  return hipGetLastError();
}

template <int MF>
hipError_t launch_general(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_i8_kernel<MF, 2, 4, 8>), dim3((unsigned)((a.N + 31) / 32)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

// Workspace of the split path: a fixed block of kCounters arrival counters
// (one per 64-row block; zero on entry, left zero by the last arriver), then
// the int32 partial sums [splits][M][N]. The counters sit at the same place
// for every shape, so one workspace serves any sequence of calls on a stream.
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = gemv_splits(M, N, K);
  if (s == 1) return 0;
  return (size_t)kCounters * sizeof(int32_t) + (size_t)(s * M * N) * sizeof(int32_t);
}

const char* decode_kernel_name(int64_t M, int64_t N, int64_t K) {
  static const char* gen[4] = {"gemv_i8_kernel<1, 2, 4, 8>", "gemv_i8_kernel<2, 2, 4, 8>",
                               "gemv_i8_kernel<3, 2, 4, 8>", "gemv_i8_kernel<4, 2, 4, 8>"};
  const int mf = gemv_mf(M);
  if (K % 128 != 0) return gen[mf - 1];
  const GemvCfg c = gemv_cfg(M, N, K);
  if (mf == 1) return c.ns == 4 ? "gemv_dma_kernel<1, 4>" : "gemv_dma_kernel<1, 8>";
  if (mf == 2) return c.ns == 4 ? "gemv_dma_kernel<2, 4>" : "gemv_dma_kernel<2, 6>";
  return mf == 3 ? "gemv_dma_kernel<3, 5>" : "gemv_dma_kernel<4, 5>";
}

hipError_t launch_decode_mm(const GemmArgs& a, void* workspace, size_t ws_bytes, int num_cus,
                            hipStream_t stream) {
  (void)num_cus;
  const int mf = gemv_mf(a.M);
  if (a.K % 128 != 0) {
    switch (mf) {
      case 1: return launch_general<1>(a, stream);
      case 2: return launch_general<2>(a, stream);
      case 3: return launch_general<3>(a, stream);
      default: return launch_general<4>(a, stream);
    }
  }
  const GemvCfg c = gemv_cfg(a.M, a.N, a.K);
  int splits = c.splits;
  const size_t need = decode_workspace_bytes(a.M, a.N, a.K);
  if (splits > 1 && (workspace == nullptr || ws_bytes < need)) splits = 1;
  int32_t* counters = static_cast<int32_t*>(workspace);
  int32_t* part = counters ? counters + kCounters : nullptr;
  switch (mf) {
    case 1:
      return c.ns == 4 ? launch_dma<1, 4>(a, splits, part, counters, stream)
                       : launch_dma<1, 8>(a, splits, part, counters, stream);
    case 2:
      return c.ns == 4 ? launch_dma<2, 4>(a, splits, part, counters, stream)
                       : launch_dma<2, 6>(a, splits, part, counters, stream);
    case 3: return launch_dma<3, 5>(a, splits, part, counters, stream);
    default: return launch_dma<4, 5>(a, splits, part, counters, stream);
  }
}

}  // namespace w8a8
