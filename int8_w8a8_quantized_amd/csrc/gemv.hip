// Decode-shaped (M <= 128) int8 GEMM: weight-streaming kernels.
//
// Same product and fused epilogue as the prefill GEMM ("[SGLang] W4A8, W8A8,
// W4A4: 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3-§4), but with a handful of
// token rows the time is reading the N x K int8 weight from HBM once. Two
// facts measured on MI355X shape the kernels:
//  - HBM streams at full rate when each wave instruction reads whole 128-byte
//    lines (8 rows x 128 bytes); the MFMA operand order (16 rows x 64 bytes)
//    reaches only about 60-70% of it;
//  - the loaded latency is several microseconds, so a CU needs on the order
//    of 100+ KiB of weight loads in flight. LDS (160 KiB, shared with the
//    activation stages) cannot hold that much; the register file can.
//
// Main kernel, gemv_reg_kernel (K a multiple of 128): a workgroup of W waves
// owns 16 * RG weight rows; the waves split K into interleaved 128-byte steps.
// Each wave keeps a ring of U steps of loads in flight in registers: the
// weight rows and the activation rows as whole lines (2 * RG and 2 * MF
// instructions per step; activation rows past M repeat row M - 1, so they
// cost cache hits, not HBM). A step's lines go through a 2 KiB-per-16-rows
// LDS buffer of the wave to reach operand order (one 16-byte write and one
// 16-byte read per lane per 8 rows; XOR-swizzled chunks keep both
// conflict-free), then v_mfma_i32_16x16x64_i8 accumulates. At the end the
// waves' partial tiles are added in LDS and the epilogue, whose per-row /
// per-column operands were loaded before the K loop, writes out.
//
// Shared-activation kernel, gemv_shared_kernel (K a multiple of 128; M > 16
// with many weight rows or a long K): a workgroup of W waves (4, or 7) owns
// 16 W weight rows; one activation stage per K step serves all of them
// through LDS. With a long K the workgroups take K ranges and a second kernel
// adds them.
//
// General kernel (any K that is a multiple of 16), gemv_i8_kernel: operands
// go straight from memory into MFMA registers, as described above it.

#include <algorithm>

#include "gemm_common.h"
#include "quant_common.h"

namespace w8a8 {

__device__ __forceinline__ int64_t gemv_min(int64_t a, int64_t b) { return a < b ? a : b; }

// Chunk position of logical 16-byte chunk c of an 8-chunk (128-byte) row r:
// distinct banks for 16-byte reads of 8 (32-bank view) or 16 (64-bank view)
// consecutive rows at one chunk.
__device__ __forceinline__ int gemv_swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// Epilogue operands of the tile elements a thread stores, loaded before the K
// loop. Element e of a wave's accumulator tile (RG row groups x MF token
// blocks of 16 x 16): gf = e / 256 -> row group gf / MF, token block gf % MF;
// register r = (e / 64) % 4; lane l = e % 64 -> weight row 16 * (gf / MF) +
// l % 16, token 16 * (gf % MF) + 4 * (l / 16) + r (the MFMA result layout).
template <int MF, int EP>
struct GemvEpi {
  EpiRow er[EP];
  EpiCol ec[EP];
  int64_t n[EP];
  __device__ __forceinline__ void load(const GemmArgs& a, int64_t n0, int first, int stride, int per) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int e = first + stride * j;
      const int gf = e >> 8, r = (e >> 6) & 3, l = e & 63;
      const int64_t nn = n0 + 16 * (gf / MF) + (l & 15);
      const int64_t m = 16 * (gf % MF) + 4 * (l >> 4) + r;
      er[j].ok = e < per && m < a.M;
      const int64_t mm = er[j].ok ? m : 0;
      er[j].out_row = mm;
      er[j].sx = a.s_x[a.sx_per_token ? mm : 0];
      er[j].zp = *(a.azp_mode == 1 ? a.zp + mm : reinterpret_cast<const int32_t*>(a.s_x));
      ec[j] = load_col(a, nn, a.s_w, a.bias);  // a row past N is marked not ok
      n[j] = nn;
    }
  }
};

// ---------------------------------------------------------------- main kernel
template <int MF, int RG, int W, int U>
__global__ __launch_bounds__(W * 64) void gemv_reg_kernel(GemmArgs a) {
  constexpr int BN = 16 * RG, BK = 128;
  constexpr int PER = RG * MF * 256;  // accumulator ints of one wave
  // The activation travels as whole lines too and is transposed in LDS
  // (16 * MF more rows in the wave's buffer): fragment-order loads (16 rows x
  // 64 bytes per instruction) miss L1 at a third of the line rate, and with
  // 16 weight rows per workgroup every CU reads the whole activation.
  constexpr int XR = 16 * MF;
  constexpr int TB = (BN + XR) * BK;  // the wave's transpose buffer: weight rows, then token rows
  constexpr int SM = (W * TB > W * PER * 4) ? W * TB : W * PER * 4;
  constexpr int EP = (PER + W * 64 - 1) / (W * 64);
  __shared__ __attribute__((aligned(1024))) int8_t smem[SM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int nsteps = (int)(a.K / BK);
  const int nkw = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;  // this wave's steps
  int8_t* tb = smem + wave * TB;

  // weight lines: instruction h reads rows 8h .. 8h+7 (lane l: row 8h + l/8,
  // bytes 16 (l%8) .. +15 of the step); rows past N repeat row N-1
  const int8_t* wsrc[2 * RG];
#pragma unroll
  for (int h = 0; h < 2 * RG; ++h)
    wsrc[h] = a.B + gemv_min(n0 + 8 * h + (lane >> 3), a.N - 1) * a.ldb + (lane & 7) * 16;
  // activation lines, 2 * MF instructions per step: instruction h reads token
  // rows 8h .. 8h+7 (lane l: row 8h + l/8, bytes 16 (l%8) .. +15); rows past
  // M repeat row M-1
  const int8_t* asrc[2 * MF];
#pragma unroll
  for (int h = 0; h < 2 * MF; ++h)
    asrc[h] = a.A + gemv_min(8 * h + (lane >> 3), a.M - 1) * a.lda + (lane & 7) * 16;

  GemvEpi<MF, EP> epi;
  epi.load(a, n0, tid, W * 64, PER);

  u32x4 wr[U][2 * RG], ar[U][2 * MF];
  // Loads of the wave's step j into ring slot u; a step past the end reloads
  // the last one (a cache hit), so every slot issues the same loads and the
  // compiler's in-order wait counts stay exact.
  auto issue = [&](int u, int j) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)(wave + W * min(j, nkw - 1)) * BK;
#pragma unroll
    for (int h = 0; h < 2 * RG; ++h)
      wr[u][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[h] + k0));
#pragma unroll
    for (int h = 0; h < 2 * MF; ++h) ar[u][h] = *reinterpret_cast<const u32x4*>(asrc[h] + k0);
  };
  i32x4 acc[MF][RG];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[f][g] = i32x4{0, 0, 0, 0};

  if (nkw > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, u);
  }
  for (int i0 = 0; i0 < nkw; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < nkw) {
        // weight and token lines -> operand order through the wave's LDS
        // buffer (the wave's LDS accesses execute in order, so no wait is
        // needed between this step's writes and reads, nor against the
        // previous step's reads)
#pragma unroll
        for (int h = 0; h < 2 * RG; ++h) {
          const int row = 8 * h + (lane >> 3);
          *reinterpret_cast<u32x4*>(tb + row * BK + (((lane & 7) ^ gemv_swz(row)) * 16)) = wr[u][h];
        }
#pragma unroll
        for (int h = 0; h < 2 * MF; ++h) {
          const int row = BN + 8 * h + (lane >> 3);
          *reinterpret_cast<u32x4*>(tb + row * BK + (((lane & 7) ^ gemv_swz(row)) * 16)) = ar[u][h];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int c = 4 * kb + (lane >> 4);
          i32x4 xf[MF];
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            const int row = BN + 16 * f + (lane & 15);
            xf[f] = *reinterpret_cast<const i32x4*>(tb + row * BK + ((c ^ gemv_swz(row)) * 16));
          }
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            const int row = 16 * g + (lane & 15);
            const i32x4 wf = *reinterpret_cast<const i32x4*>(tb + row * BK + ((c ^ gemv_swz(row)) * 16));
#pragma unroll
            for (int f = 0; f < MF; ++f) acc[f][g] = mfma16x16x64(xf[f], wf, acc[f][g]);
          }
        }
      }
      issue(u, i0 + u + U);
    }
  }

  // add the waves' partial tiles
  __syncthreads();
  int32_t* red = reinterpret_cast<int32_t*>(smem);
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave * PER + (g * MF + f) * 256 + r * 64 + lane] = acc[f][g][r];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EP; ++j) {
    const int e = tid + W * 64 * j;
    if (e >= PER) continue;
    int v = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[w * PER + e];
    epilogue_store(a, epi.er[j], epi.ec[j], epi.n[j], v);
  }
}

// ---------------------------------------------- shared-activation kernel
// For M > 16 with many weight rows or a long K. The L1 fill of a CU (HBM and
// L2 traffic together) is the limit there: the register kernel's 16-row
// workgroups each read the whole activation, four times the weight bytes at
// M = 64. Here the 4 waves of a workgroup own 16 weight rows each and walk
// the same K steps, so one activation stage (16 * MF rows x 128 bytes, whole
// lines, loaded cooperatively into registers with the weights) serves 64
// weight rows: it is written to a double-buffered LDS stage and, after a
// barrier, every wave reads its fragments there. Weight lines ride each
// wave's register ring and LDS transpose as in the register kernel. K is cut
// into `splits` ranges, one per workgroup. With one range (DIRECT) the
// epilogue runs in the kernel; otherwise each workgroup stores its int32 tile
// in accumulator order (256 contiguous bytes per wave instruction) to the
// caller's workspace, and gemv_reduce_kernel adds the ranges and applies the
// epilogue. The stage buffer written at step i was last read at step i - 2,
// before every wave passed the barrier of step i - 1.
constexpr int kSharedWaves = 4;

// W waves of 16 weight rows each; the split form (not DIRECT) always has
// kSharedWaves, the layout gemv_reduce_kernel reads.
template <int MF, int U, bool DIRECT, int W>
__global__ __launch_bounds__(W * 64) void gemv_shared_kernel(GemmArgs a, int splits, int steps_per_split,
                                                             int32_t* __restrict__ part) {
  static_assert(DIRECT || W == kSharedWaves, "the reduction reads kSharedWaves tiles per row block");
  constexpr int BK = 128, XR = 16 * MF;
  constexpr int AI = XR / 8;            // activation line instructions per step
  constexpr int AQ = (AI + W - 1) / W;  // per wave (the last may repeat)
  constexpr int PER = MF * 256;         // accumulator ints of one wave
  __shared__ __attribute__((aligned(1024))) int8_t abuf[2][XR * BK];
  __shared__ __attribute__((aligned(1024))) int8_t tbuf[W][16 * BK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int64_t n0 = (int64_t)rb * 16 * W + 16 * wave;  // this wave's first weight row
  const int nsteps = (int)(a.K / BK);
  const int s_begin = sp * steps_per_split;
  const int nk = max(min(nsteps, s_begin + steps_per_split) - s_begin, 0);
  int8_t* tb = tbuf[wave];

  const int8_t* wsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    wsrc[h] = a.B + gemv_min(n0 + 8 * h + (lane >> 3), a.N - 1) * a.ldb + (lane & 7) * 16;
  // activation line instruction j: stage rows 8j .. 8j+7 (rows past M repeat row M-1)
  const int8_t* asrc[AQ];
  int adst[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int j = min(wave * AQ + q, AI - 1);
    const int row = 8 * j + (lane >> 3);
    asrc[q] = a.A + gemv_min(row, a.M - 1) * a.lda + (lane & 7) * 16;
    adst[q] = row * BK + (((lane & 7) ^ gemv_swz(row)) * 16);
  }
  // DIRECT (one K range): the epilogue's operands, loaded before the K loop
  // (lane holds tokens 16f + 4*(lane/16) + r of weight row n0 + lane%16)
  const int64_t n = n0 + (lane & 15);
  EpiCol col;
  EpiRow er[MF][4];
  if (DIRECT) {
    col = load_col(a, n, a.s_w, a.bias);
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 16 * f + 4 * (lane >> 4) + r;
        er[f][r].ok = m < a.M;
        const int64_t mm = er[f][r].ok ? m : 0;
        er[f][r].out_row = mm;
        er[f][r].sx = a.s_x[a.sx_per_token ? mm : 0];
        er[f][r].zp = *(a.azp_mode == 1 ? a.zp + mm : reinterpret_cast<const int32_t*>(a.s_x));
      }
  }
  u32x4 wr[U][2], xr[U][AQ];
  // step j of this range into ring slot u; past the end: a reload of the last step
  auto issue = [&](int u, int j) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)(s_begin + min(j, nk - 1)) * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wr[u][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[h] + k0));
#pragma unroll
    for (int q = 0; q < AQ; ++q) xr[u][q] = *reinterpret_cast<const u32x4*>(asrc[q] + k0);
  };
  i32x4 acc[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) acc[f] = i32x4{0, 0, 0, 0};
  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, u);
  }
  for (int i0 = 0; i0 < nk; i0 += U) {  // nk is the same for every wave of the workgroup
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      if (i < nk) {
        int8_t* ab = abuf[i & 1];
#pragma unroll
        for (int q = 0; q < AQ; ++q) *reinterpret_cast<u32x4*>(ab + adst[q]) = xr[u][q];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 8 * h + (lane >> 3);
          *reinterpret_cast<u32x4*>(tb + row * BK + (((lane & 7) ^ gemv_swz(row)) * 16)) = wr[u][h];
        }
        // the stage is complete once every wave's writes have landed (no vmcnt
        // wait here: the ring's later loads stay in flight)
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int c = 4 * kb + (lane >> 4);
          const int wrow = lane & 15;
          const i32x4 wf = *reinterpret_cast<const i32x4*>(tb + wrow * BK + ((c ^ gemv_swz(wrow)) * 16));
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            const int xrow = 16 * f + (lane & 15);
            const i32x4 xf = *reinterpret_cast<const i32x4*>(ab + xrow * BK + ((c ^ gemv_swz(xrow)) * 16));
            acc[f] = mfma16x16x64(xf, wf, acc[f]);
          }
        }
      }
      issue(u, i + U);
    }
  }
  if (DIRECT) {
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) epilogue_store(a, er[f][r], col, n, acc[f][r]);
    return;
  }
  // lane holds tokens 16f + 4*(lane/16) + r of weight row n0 + lane%16
  int32_t* dst = part + (((int64_t)rb * splits + sp) * W + wave) * PER + lane;
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(f * 4 + r) * 64] = acc[f][r];
}

// Sum of the K ranges' tiles and the epilogue; one thread per accumulator
// element, in the order gemv_shared_kernel stored them.
template <int MF>
__global__ __launch_bounds__(256) void gemv_reduce_kernel(GemmArgs a, int splits,
                                                          const int32_t* __restrict__ part) {
  constexpr int W = kSharedWaves, PER = MF * 256;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over row blocks x waves x PER
  const int64_t rbw = e / PER;                                 // row block * W + wave
  const int pe = (int)(e % PER);
  const int64_t rb = rbw / W;
  const int wave = (int)(rbw % W);
  const int f = pe / 256, r = (pe / 64) % 4, lane = pe % 64;
  const int64_t n = rb * 16 * W + 16 * wave + (lane & 15);
  const int64_t m = 16 * f + 4 * (lane >> 4) + r;
  if (n >= a.N || m >= a.M) return;
  // the epilogue operands go out first, so their round trip overlaps the
  // partial tiles' instead of following it
  EpiRow er;
  er.ok = true;
  er.out_row = m;
  er.sx = a.s_x[a.sx_per_token ? m : 0];
  er.zp = *(a.azp_mode == 1 ? a.zp + m : reinterpret_cast<const int32_t*>(a.s_x));
  const EpiCol col = load_col(a, n, a.s_w, a.bias);
  const int32_t* src = part + (rb * splits * W + wave) * PER + pe;
  int32_t pv[8];
  int v = 0;
  for (int s0 = 0; s0 < splits; s0 += 8) {  // splits <= 8 in practice: one batch of loads
    // ranges past the last one reload it (a valid address) and are not added
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = src[(int64_t)min(s0 + j, splits - 1) * W * PER];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += (s0 + j < splits) ? pv[j] : 0;
  }
  epilogue_store(a, er, col, n, v);
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
  // A lane whose 16 bytes start at or past K (the tail of a K that is not a
  // multiple of 64) reads the start of its rows instead, so no load leaves a
  // row; its activation is zero, so the product does not depend on it.
  auto load_step = [&](int u, int step) __attribute__((always_inline)) {
    const bool live = step < nsteps;
    const int64_t k = (int64_t)(live ? step : 0) * 64;
    const int64_t kw = k + kgrp < a.K ? k : 0;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      wb[u][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[j] + kw));
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

// ------------------------------------ fused activation quantisation
// gemv_fused_kernel: the register kernel's weight stream (M = 1 token block)
// on an activation the workgroup quantises itself, per token and symmetric,
// so one launch does the work of the quantiser and the decode GEMM. It
// serves M <= kFusedRows and M * K <= kFusedElems: each thread loads its
// share of the bf16 rows (at most kFusedElems / 8 / threads 16-byte chunks);
// the rows' absmax is reduced over the workgroup and each chunk is encoded by
// the quantiser's own code path (identical codes and scales). The codes stay
// in LDS for the whole K loop, rows padded by 16 bytes so the fragment reads
// of the two rows fall in different banks. Every workgroup reads the same
// bf16 rows (cache hits after the first) and computes the same codes;
// workgroup 0 also writes them and the scales out. The prologue is paid by
// every workgroup before its K loop can start, so the launch table uses this
// kernel only where that costs less than a separate quantiser launch.
constexpr int kFusedRows = 2;
constexpr int kFusedElems = 16384;

template <int RG, int W, int U>
__global__ __launch_bounds__(W * 64) void gemv_fused_kernel(GemmArgs a, const uint16_t* __restrict__ x,
                                                            int64_t ldx, int8_t* __restrict__ xq,
                                                            int64_t ldq, float* __restrict__ sx) {
  constexpr int BN = 16 * RG, BK = 128, NT = W * 64;
  constexpr int PER = RG * 256;  // accumulator ints of one wave
  constexpr int TB = BN * BK;    // the wave's weight transpose buffer
  constexpr int SM = (W * TB > W * PER * 4) ? W * TB : W * PER * 4;
  constexpr int EP = (PER + NT - 1) / NT;
  constexpr int CHX = kFusedElems / 8 / NT;  // activation chunks per thread, at most
  __shared__ __attribute__((aligned(1024))) int8_t smem[SM];
  __shared__ __attribute__((aligned(16))) int8_t xs[kFusedElems + 16 * kFusedRows];
  __shared__ float red_max[kFusedRows][W];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int M = (int)a.M, K = (int)a.K;
  const int kc = K >> 3;        // 16-byte chunks per row
  const int xst = K + 16;       // LDS row stride of the codes
  const int nsteps = K / BK;
  const int nkw = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  int8_t* tb = smem + wave * TB;

  // the activation chunks: chunk j = c * NT + tid of the M x kc grid, row
  // j / kc (M <= 2: one comparison); chunks past the grid read chunk 0
  uint4 xv[CHX];
#pragma unroll
  for (int c = 0; c < CHX; ++c) {
    const int j0 = c * NT + tid;
    const int j = j0 < M * kc ? j0 : 0;
    const int m = j >= kc;
    xv[c] = ld16(x + (int64_t)m * ldx + (int64_t)(j - m * kc) * 8);
  }
  // per-row absmax over the workgroup
  float am[kFusedRows] = {0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < CHX; ++c) {
    const int j = c * NT + tid;
    const int m = j >= kc;
    float v = 0.0f;
    absmax8(xv[c], v);
    const bool in = j < M * kc;
#pragma unroll
    for (int r = 0; r < kFusedRows; ++r) am[r] = (in && m == r) ? max_ieee(am[r], v) : am[r];
  }
  __builtin_amdgcn_sched_barrier(0);
  // The weight ring goes out once this thread's activation chunks have
  // arrived: issued first, the activation loads would queue behind every
  // CU's weight loads. The ring then overlaps the reductions, the encoding
  // and the two barriers.
  // the weight ring, as in the register kernel (rows past N repeat row N-1)
  const int8_t* wsrc[2 * RG];
#pragma unroll
  for (int h = 0; h < 2 * RG; ++h)
    wsrc[h] = a.B + gemv_min(n0 + 8 * h + (lane >> 3), a.N - 1) * a.ldb + (lane & 7) * 16;
  u32x4 wr[U][2 * RG];
  // Step j of this wave (past its last step: the last one again; a wave with
  // no steps reads step nsteps - 1 and never uses it). The prefill is
  // unconditional, so the compiler's wait counts for the activation loads
  // above see the ring as always in flight and do not wait for it.
  auto issue = [&](int u, int j) __attribute__((always_inline)) {
    const int step = min(wave + W * max(min(j, nkw - 1), 0), nsteps - 1);
    const int64_t k0 = (int64_t)step * BK;
#pragma unroll
    for (int h = 0; h < 2 * RG; ++h)
      wr[u][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[h] + k0));
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, u);
  GemvEpi<1, EP> epi;  // s_x is not read: the scales are set below
  epi.load(a, n0, tid, NT, PER);

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < kFusedRows; ++r) am[r] = wave_extreme<true>(am[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kFusedRows; ++r) red_max[r][wave] = am[r];
  }
  // LDS only: the weight loads stay in flight across this barrier
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  RowParams rp[kFusedRows];
#pragma unroll
  for (int r = 0; r < kFusedRows; ++r) {
    float v = red_max[r][0];
#pragma unroll
    for (int w = 1; w < W; ++w) v = max_ieee(v, red_max[r][w]);
    rp[r] = row_params<kDynSym>(0.0f, v, nullptr, nullptr);
  }

  // codes into LDS (and out, from workgroup 0)
  const bool writer = blockIdx.x == 0;
#pragma unroll
  for (int c = 0; c < CHX; ++c) {
    const int j = c * NT + tid;
    if (j < M * kc) {
      const int m = j >= kc;
      const RowParams q = m ? rp[1] : rp[0];
      const uint2 code = codes8<kDynSym>(xv[c], q);
      const int col = (j - m * kc) * 8;
      *reinterpret_cast<uint2*>(xs + m * xst + col) = code;
      if (writer) *reinterpret_cast<uint2*>(xq + (int64_t)m * ldq + col) = code;
    }
  }
  if (writer && tid < M) sx[tid] = tid == 0 ? rp[0].s : rp[1].s;
#pragma unroll
  for (int j = 0; j < EP; ++j) {
    const int64_t m = epi.er[j].out_row;  // 0 for elements outside the output
    epi.er[j].sx = m == 0 ? rp[0].s : rp[1].s;
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // K loop: weight lines -> operand order through the wave's LDS buffer; the
  // activation fragments straight from the resident codes (token rows past M
  // repeat row M-1)
  const int xrow = min(lane & 15, M - 1);
  const int8_t* xbase = xs + xrow * xst + (lane >> 4) * 16;
  i32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = i32x4{0, 0, 0, 0};
  for (int i0 = 0; i0 < nkw; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < nkw) {
#pragma unroll
        for (int h = 0; h < 2 * RG; ++h) {
          const int row = 8 * h + (lane >> 3);
          *reinterpret_cast<u32x4*>(tb + row * BK + (((lane & 7) ^ gemv_swz(row)) * 16)) = wr[u][h];
        }
        const int k0 = (wave + W * (i0 + u)) * BK;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int c = 4 * kb + (lane >> 4);
          const i32x4 xf = *reinterpret_cast<const i32x4*>(xbase + k0 + 64 * kb);
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            const int row = 16 * g + (lane & 15);
            const i32x4 wf = *reinterpret_cast<const i32x4*>(tb + row * BK + ((c ^ gemv_swz(row)) * 16));
            acc[g] = mfma16x16x64(xf, wf, acc[g]);
          }
        }
      }
      issue(u, i0 + u + U);
    }
  }

  // add the waves' partial tiles
  __syncthreads();
  int32_t* red = reinterpret_cast<int32_t*>(smem);
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * PER + g * 256 + r * 64 + lane] = acc[g][r];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EP; ++j) {
    const int e = tid + NT * j;
    if (e >= PER) continue;
    int v = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[w * PER + e];
    epilogue_store(a, epi.er[j], epi.ec[j], epi.n[j], v);
  }
}

namespace {

// Launch shape of the decode kernels, from sweeps over the Llama-3-8B decode
// linears (M in {1, 8, 32, 64}, K x N in {4096 x 6144, 4096 x 4096,
// 4096 x 28672, 14336 x 4096}) timed as graph replays with the weights
// rotated over 1 GiB:
//  - M <= 16: the register kernel, 16 rows per workgroup; 4 waves split K,
//    2 once there are more than 512 row groups (the waves then live long
//    enough); from M = 12 on with more than 8192 weight rows, the
//    shared-activation kernel below instead;
//  - M > 16 with more than 8192 weight rows: the shared-activation kernel
//    over the whole K with the epilogue in the kernel (its 64-row workgroups
//    fill the chip; 4096 x 28672: 25.5 / 30.3 us at M = 32 / 64, where an
//    LDS ring for the weights as well took 28.1 / 32.7; 4096 x 14336 at
//    M = 17 / 64: 13.7 / 17.4 us against 17.9 / 29.8 for the register
//    kernel, whose 16-row workgroups each read the whole activation), with
//    7 waves (112 rows) from M = 33 on where that makes whole rounds of 256
//    workgroups (4096 x 28672 at M = 48 / 64: 27.3 / 29.3 us against 28.4 /
//    31.3; 6 or 8 waves, or 7 with a partial round, are slower);
//  - M > 16, 64 steps of K or more and a workspace: the shared-activation
//    kernel over about 256 workgroups (K ranges of at least 16 steps), then
//    the reduction;
//  - the shared kernel keeps 4 steps in flight per wave (14336 x 4096 with
//    the reduction: 14.8 / 18.1 us at M = 32 / 64; 8 and 6 steps took
//    16.9 / 20.4);
//  - otherwise the register kernel, with 32 rows per workgroup when 16-row
//    groups would need between one and two workgroups per CU (a half-empty
//    second round costs more than the larger tile);
//  - a short K (at most 40 steps) over 256 - 512 row groups leaves one
//    workgroup per CU: there 8 waves with a ring of 2 (M <= 16) or 1 steps
//    beat 4 waves with 4 (0.4 - 1.4 us per launch at K = 4096 - 5120).
enum class GemvKind { kReg, kShared, kGeneral, kTile };  // kTile: the MFMA tile kernel
struct GemvCfg {
  GemvKind kind;
  int mf, rg, w, u;  // u: ring steps in flight per wave
  int splits;        // K ranges of the shared kernel (1: the epilogue runs in it)
};

// Token blocks of 16: up to 4 on every decode path, 5 - 8 (M = 65 - 128) on
// the split shared kernel only.
int gemv_mf(int64_t M) { return (int)std::min<int64_t>((M + 15) / 16, 8); }

// The shared kernel's K ranges for this shape (0: not used).
int shared_splits(int64_t M, int64_t N, int64_t K) {
  if (gemv_mf(M) == 1 || K % 128 != 0 || N > 8192) return 0;  // N > 8192: one K range
  const int64_t nsteps = K / 128, rbs = (N + 63) / 64;
  if (gemv_mf(M) > 4) {
    // M = 65 - 128: ranges of at least 8 steps (65 x 14336 x 4096: 21.3 us
    // in 4 ranges against 57.8 on the MFMA tiles, 65 x 4096 x 4096 12.4
    // against 20.5; 112 x 8192 x 2048: 15.0 in 8 ranges against 37.6)
    const int64_t s = std::min<int64_t>(std::max<int64_t>(256 / rbs, 1), std::min<int64_t>(8, nsteps / 8));
    return s >= 2 ? (int)s : 0;
  }
  if (nsteps < 64) return 0;
  const int64_t s = std::min<int64_t>(std::max<int64_t>(256 / rbs, 1), std::min<int64_t>(8, nsteps / 16));
  return s >= 2 ? (int)s : 0;
}

size_t shared_workspace_bytes(int64_t M, int64_t N, int splits) {
  const int64_t rbs = (N + 63) / 64;
  return (size_t)splits * rbs * kSharedWaves * gemv_mf(M) * 256 * sizeof(int32_t);
}

// Every register-kernel instance the table below can choose:
// (token blocks, row groups, waves, ring steps).
#define W8A8_GEMV_REG_INSTANCES(X)                                                    \
  X(1, 1, 4, 4) X(1, 1, 2, 4) X(1, 1, 8, 2) X(1, 2, 8, 2) X(2, 1, 4, 4) X(2, 1, 8, 1) \
  X(2, 2, 4, 4) X(2, 2, 8, 1) X(3, 1, 4, 4) X(3, 1, 8, 1) X(3, 2, 4, 3) X(4, 1, 4, 4) \
  X(4, 1, 8, 1) X(4, 2, 4, 3) X(4, 2, 8, 1)

GemvCfg gemv_cfg(int64_t M, int64_t N, int64_t K, size_t ws_bytes) {
  const int mf = gemv_mf(M);
  if (mf > 4) {  // M = 65 - 128: K ranges of the shared kernel, else the MFMA tiles
    const int s = shared_splits(M, N, K);
    if (s > 0 && ws_bytes >= shared_workspace_bytes(M, N, s)) return {GemvKind::kShared, mf, 1, kSharedWaves, 4, s};
    return {GemvKind::kTile, mf, 0, 0, 0, 0};
  }
  if (K % 128 != 0) return {GemvKind::kGeneral, mf, 2, 4, 8, 1};
  const int64_t groups = (N + 15) / 16;
  // A short K (at most 40 steps) over 256 - 512 row groups leaves one
  // workgroup per CU: 8 waves with a shallower ring then beat 4 waves with a
  // deep one (measured 0.4 - 1.4 us per launch at K = 4096 - 5120; with a
  // longer K, or more or fewer groups, the 4-wave table is as fast or faster).
  const bool short_k = K / 128 <= 40 && groups >= 256 && groups <= 512;
  const int rg_short = groups > 256 ? 2 : 1;
  if (mf == 1) {
    if (short_k) return {GemvKind::kReg, 1, rg_short, 8, 2, 1};
    // from M = 12 on, wide weights read the activation once per 64 rows
    // (bf16 out with bias: 16 x 4096 x 28672 23.5 us against 24.8, 16 x
    // 14336 x 28672 63.8 against 72.8; at M = 8 the two are even)
    if (M >= 12 && N > 8192) return {GemvKind::kShared, 1, 1, kSharedWaves, 4, 1};
    // 2 waves once there are more than 512 row groups (8 x 4096 x 14336:
    // 13.3 us against 15.0 with 4)
    return {GemvKind::kReg, 1, 1, groups > 512 ? 2 : 4, 4, 1};
  }
  if (N > 8192) {
    // one K range over 64-row workgroups, or 112-row ones (7 waves) from
    // M = 33 on when those make whole rounds over the CUs (4096 x 28672:
    // 256 workgroups instead of 448 sharing each activation stage)
    const bool seven = mf >= 3 && ((N + 111) / 112) % 256 == 0;
    return {GemvKind::kShared, mf, 1, seven ? 7 : kSharedWaves, 4, 1};
  }
  const int s = shared_splits(M, N, K);
  if (s > 0 && ws_bytes >= shared_workspace_bytes(M, N, s)) return {GemvKind::kShared, mf, 1, kSharedWaves, 4, s};
  if (short_k && !(mf == 3 && rg_short == 2)) return {GemvKind::kReg, mf, rg_short, 8, 1, 1};
  if (groups > 256 && groups <= 512) return {GemvKind::kReg, mf, 2, 4, mf == 2 ? 4 : 3, 1};
  return {GemvKind::kReg, mf, 1, 4, 4, 1};
}

template <int MF, int RG, int W, int U>
hipError_t launch_reg(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.N + 16 * RG - 1) / (16 * RG);
  hipLaunchKernelGGL((gemv_reg_kernel<MF, RG, W, U>), dim3((unsigned)blocks), dim3(W * 64), 0, stream, a);
  return hipGetLastError();
}

template <int MF, int U>
hipError_t launch_shared(const GemmArgs& a, int splits, int waves, int32_t* part, hipStream_t stream) {
  const int64_t nsteps = a.K / 128;
  const int sps = (int)((nsteps + splits - 1) / splits);
  if (splits == 1) {  // one K range: the epilogue runs in the kernel, no workspace
    if (waves == 7) {
      hipLaunchKernelGGL((gemv_shared_kernel<MF, U, true, 7>), dim3((unsigned)((a.N + 111) / 112)), dim3(7 * 64),
                         0, stream, a, 1, sps, nullptr);
    } else {
      hipLaunchKernelGGL((gemv_shared_kernel<MF, U, true, kSharedWaves>), dim3((unsigned)((a.N + 63) / 64)),
                         dim3(kSharedWaves * 64), 0, stream, a, 1, sps, nullptr);
    }
    return hipGetLastError();
  }
  const int64_t rbs = (a.N + 63) / 64;
  hipLaunchKernelGGL((gemv_shared_kernel<MF, U, false, kSharedWaves>), dim3((unsigned)(rbs * splits)),
                     dim3(kSharedWaves * 64), 0, stream, a, splits, sps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t elems = rbs * kSharedWaves * MF * 256;
  hipLaunchKernelGGL((gemv_reduce_kernel<MF>), dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, stream,
                     a, splits, part);
  return hipGetLastError();
}

// 5 - 8 token blocks: the split form only (its epilogue runs in the
// reduction, so the kernel holds no per-row epilogue operands).
template <int MF>
hipError_t launch_shared_split(const GemmArgs& a, int splits, int32_t* part, hipStream_t stream) {
  const int64_t nsteps = a.K / 128, rbs = (a.N + 63) / 64;
  const int sps = (int)((nsteps + splits - 1) / splits);
  hipLaunchKernelGGL((gemv_shared_kernel<MF, 4, false, kSharedWaves>), dim3((unsigned)(rbs * splits)),
                     dim3(kSharedWaves * 64), 0, stream, a, splits, sps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t elems = rbs * kSharedWaves * MF * 256;
  hipLaunchKernelGGL((gemv_reduce_kernel<MF>), dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, stream, a,
                     splits, part);
  return hipGetLastError();
}

template <int MF>
hipError_t launch_general(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_i8_kernel<MF, 2, 4, 8>), dim3((unsigned)((a.N + 31) / 32)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = shared_splits(M, N, K);
  return s > 0 ? shared_workspace_bytes(M, N, s) : 0;
}

const char* decode_kernel_name(int64_t M, int64_t N, int64_t K, size_t ws_bytes) {
  const GemvCfg c = gemv_cfg(M, N, K, ws_bytes);
  switch (c.kind) {
    case GemvKind::kGeneral: {
      static const char* gen[4] = {"gemv_i8_kernel<1, 2, 4, 8>", "gemv_i8_kernel<2, 2, 4, 8>",
                                   "gemv_i8_kernel<3, 2, 4, 8>", "gemv_i8_kernel<4, 2, 4, 8>"};
      return gen[c.mf - 1];
    }
    case GemvKind::kTile: return scaled_mm_kernel_name(M, N, K);
    case GemvKind::kShared: {
      static const char* split[8] = {"gemv_shared_kernel<1, 4, false, 4>", "gemv_shared_kernel<2, 4, false, 4>",
                                     "gemv_shared_kernel<3, 4, false, 4>", "gemv_shared_kernel<4, 4, false, 4>",
                                     "gemv_shared_kernel<5, 4, false, 4>", "gemv_shared_kernel<6, 4, false, 4>",
                                     "gemv_shared_kernel<7, 4, false, 4>", "gemv_shared_kernel<8, 4, false, 4>"};
      static const char* direct[4] = {"gemv_shared_kernel<1, 4, true, 4>", "gemv_shared_kernel<2, 4, true, 4>",
                                      "gemv_shared_kernel<3, 4, true, 4>", "gemv_shared_kernel<4, 4, true, 4>"};
      static const char* direct7[4] = {"gemv_shared_kernel<1, 4, true, 7>", "gemv_shared_kernel<2, 4, true, 7>",
                                       "gemv_shared_kernel<3, 4, true, 7>", "gemv_shared_kernel<4, 4, true, 7>"};
      if (c.splits != 1) return split[c.mf - 1];
      return c.w == 7 ? direct7[c.mf - 1] : direct[c.mf - 1];
    }
    default: break;
  }
#define W8A8_REG_NAME(MF, RG, W, U) \
  if (c.mf == MF && c.rg == RG && c.w == W && c.u == U) return "gemv_reg_kernel<" #MF ", " #RG ", " #W ", " #U ">";
  W8A8_GEMV_REG_INSTANCES(W8A8_REG_NAME)
#undef W8A8_REG_NAME
  return "unknown";
}

// Where one fused launch beats the quantiser launch plus the GEMM (graph
// replays, weights rotated over 1 GiB): with at most one 16-row workgroup per
// CU (N <= 4096) and M <= 2 -- 1 x 4096 x 4096: 6.7 against 7.7 us, 2 x 4096
// x 4096: 7.5 against 8.0, 1 x 14336 x 4096: 13.8 against 14.2. With more
// workgroups each round pays the prologue again (1 x 4096 x 28672: 28.5
// against 27.1 us; 4 x 4096 x 28672: 36.3 against 24.3), and 32-row
// workgroups or more rows lose too (1 x 4096 x 6144: 9.7 against 9.3).
bool fused_linear_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= kFusedRows && N >= 1 && N <= 4096 && K % 128 == 0 && M * K <= kFusedElems;
}

namespace {
// The fused kernel takes the register kernel's launch shape for M <= 16.
template <int RG, int W, int U>
hipError_t launch_fused(const GemmArgs& a, const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldq,
                        float* s_x, hipStream_t stream) {
  const int64_t blocks = (a.N + 16 * RG - 1) / (16 * RG);
  hipLaunchKernelGGL((gemv_fused_kernel<RG, W, U>), dim3((unsigned)blocks), dim3(W * 64), 0, stream, a, x, ldx,
                     xq, ldq, s_x);
  return hipGetLastError();
}
}  // namespace

// N <= 4096 leaves two of the register kernel's launch shapes: 8 waves in
// the short-K band (N = 4081 .. 4096), 4 otherwise.
const char* fused_linear_kernel_name(int64_t M, int64_t N, int64_t K) {
  return gemv_cfg(M, N, K, 0).w == 8 ? "gemv_fused_kernel<1, 8, 2>" : "gemv_fused_kernel<1, 4, 4>";
}

hipError_t launch_fused_linear(const GemmArgs& a, const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldq,
                               float* s_x, hipStream_t stream) {
  if (!fused_linear_fits(a.M, a.N, a.K)) return hipErrorInvalidValue;
  GemmArgs f = a;
  f.A = nullptr;                 // the codes come from x
  f.s_x = a.s_w;                 // read by the epilogue set-up, then replaced
  f.sx_per_token = 0;
  f.azp_mode = 0;
  f.out_i32 = 0;
  const GemvCfg c = gemv_cfg(a.M, a.N, a.K, 0);  // the register kernel's row for M <= 16
  return c.w == 8 ? launch_fused<1, 8, 2>(f, x, ldx, xq, ldq, s_x, stream)
                  : launch_fused<1, 4, 4>(f, x, ldx, xq, ldq, s_x, stream);
}

hipError_t launch_decode_mm(const GemmArgs& a, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const GemvCfg c = gemv_cfg(a.M, a.N, a.K, workspace ? ws_bytes : 0);
  int32_t* part = static_cast<int32_t*>(workspace);
  switch (c.kind) {
    case GemvKind::kGeneral:
      switch (c.mf) {
        case 1: return launch_general<1>(a, stream);
        case 2: return launch_general<2>(a, stream);
        case 3: return launch_general<3>(a, stream);
        default: return launch_general<4>(a, stream);
      }
    case GemvKind::kTile: return launch_scaled_mm(a, stream);
    case GemvKind::kShared:
      switch (c.mf) {
        case 5: return launch_shared_split<5>(a, c.splits, part, stream);
        case 6: return launch_shared_split<6>(a, c.splits, part, stream);
        case 7: return launch_shared_split<7>(a, c.splits, part, stream);
        case 8: return launch_shared_split<8>(a, c.splits, part, stream);
        case 1: return launch_shared<1, 4>(a, c.splits, c.w, part, stream);
        case 2: return launch_shared<2, 4>(a, c.splits, c.w, part, stream);
        case 3: return launch_shared<3, 4>(a, c.splits, c.w, part, stream);
        default: return launch_shared<4, 4>(a, c.splits, c.w, part, stream);
      }
    default: break;
  }
#define W8A8_REG_LAUNCH(MF, RG, W, U) \
  if (c.mf == MF && c.rg == RG && c.w == W && c.u == U) return launch_reg<MF, RG, W, U>(a, stream);
  W8A8_GEMV_REG_INSTANCES(W8A8_REG_LAUNCH)
#undef W8A8_REG_LAUNCH
  return hipErrorInvalidValue;  // not reached: the table picks only listed instances
}

}  // namespace w8a8
