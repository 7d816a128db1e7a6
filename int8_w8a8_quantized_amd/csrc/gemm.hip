// Prefill-shaped and grouped (MoE) int8 GEMMs on CDNA4 int8 MFMA.
//
// out[t,n] = epilogue( sum_k xq[t,k] * Wq[n,k] ) -- the int8 x int8 -> int32
// product of "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴" (핵심 코드 분석
// §3) against the [out_features, in_features] weight of "vLLM INT8 W8A8 量化实战"
// (4.2), with the scale / zero-point / bias epilogue of the same page (§3-§4)
// fused into the store.
//
// Both operands are K-contiguous ("NT"). A workgroup of 4 waves owns a
// BM x BN output tile and walks K in BK-byte steps: each thread moves 16-byte
// chunks of the A and B tiles from HBM into registers, then into LDS (rows
// padded by 16 bytes so the 16-byte fragment reads of a wave hit distinct
// banks), double-buffered so the global loads of step k+1 are in flight while
// the MFMAs of step k run. Each wave computes a (BM/2) x (BN/2) sub-tile as a
// grid of 16x16 int32 accumulators with v_mfma_i32_16x16x64_i8.
//
// Tile order: workgroup ids are spread round-robin over the 8 XCDs, so the
// linear id is first remapped to give each XCD a contiguous range of tiles,
// which are then walked in groups of 8 tile-rows so that neighbouring
// workgroups share A and B tiles in that XCD's L2.
//
// The grouped variant maps each workgroup to (expert, m-tile of that
// expert's row range, n-tile) by scanning expert_offsets; rows may be
// gathered through row_ids in the A load.

#include "gemm_common.h"

namespace w8a8 {

template <int BM, int BN, int BK, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_i8_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int NT = 256;
  constexpr int WM = 2, WN = 2;
  constexpr int STRIDE = BK + 16;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KC = BK / 16;
  constexpr int A_PER_T = BM * KC / NT, B_PER_T = BN * KC / NT;
  static_assert(BM * KC % NT == 0 && BN * KC % NT == 0, "tile / thread mismatch");
  static_assert(BK % 64 == 0, "BK is a multiple of the MFMA k");

  __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- which tile
  int tn;
  int64_t row_begin, row_end;
  const int8_t* B = a.B;
  const float* sw = a.s_w;
  const uint16_t* bias = a.bias;
  if (GROUPED) {
    const int mt = blockIdx.x / tiles_n;
    tn = blockIdx.x % tiles_n;
    const int64_t T = a.M;
    int64_t cum = 0, e_found = -1;
    int64_t prev = 0;
    for (int64_t e = 0; e < a.E; ++e) {
      int64_t s0 = a.expert_offsets[e], s1 = a.expert_offsets[e + 1];
      s0 = min(max(s0, prev), T);
      s1 = min(max(s1, s0), T);
      prev = s0;
      const int64_t t_e = (s1 - s0 + BM - 1) / BM;
      if (mt < cum + t_e) {
        e_found = e;
        row_begin = s0 + (int64_t)(mt - cum) * BM;
        row_end = s1;
        break;
      }
      cum += t_e;
    }
    if (e_found < 0) return;
    B += e_found * a.N * a.ldb;
    sw += e_found * a.N;
    if (bias) bias += e_found * a.N;
  } else {
    int pid = blockIdx.x;
    const int nwg = gridDim.x;
    if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
    constexpr int GM = 8;
    const int group = pid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in_group = pid % (GM * tiles_n);
    const int tm = first_m + in_group % gsz;
    tn = in_group / gsz;
    row_begin = (int64_t)tm * BM;
    row_end = a.M;
  }
  const int64_t n_begin = (int64_t)tn * BN;

  // ---- per-thread global source pointers (fixed over K)
  const int8_t* a_src[A_PER_T];
  bool a_ok[A_PER_T];
  int a_kc[A_PER_T], a_lds[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = tid + i * NT, r = c / KC, kc = c % KC;
    const int64_t gr = row_begin + r;
    bool ok = gr < row_end;
    int64_t src = ok ? gr : 0;
    if (GROUPED && a.row_ids) {
      src = ok ? (int64_t)a.row_ids[gr] : 0;
      ok = ok && src >= 0 && src < a.M_src;
      if (!ok) src = 0;
    }
    a_src[i] = a.A + src * a.lda + kc * 16;
    a_ok[i] = ok;
    a_kc[i] = kc * 16;
    a_lds[i] = r * STRIDE + kc * 16;
  }
  const int8_t* b_src[B_PER_T];
  bool b_ok[B_PER_T];
  int b_kc[B_PER_T], b_lds[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int c = tid + i * NT, r = c / KC, kc = c % KC;
    const int64_t n = n_begin + r;
    b_ok[i] = n < a.N;
    b_src[i] = B + (b_ok[i] ? n : 0) * a.ldb + kc * 16;
    b_kc[i] = kc * 16;
    b_lds[i] = BM * STRIDE + r * STRIDE + kc * 16;
  }

  uint4 ra[A_PER_T], rb[B_PER_T];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i)
      ra[i] = (a_ok[i] && k0 + a_kc[i] < a.K) ? ld16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i)
      rb[i] = (b_ok[i] && k0 + b_kc[i] < a.K) ? ld16(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store_tile = [&](int buf) {
    int8_t* base = smem + buf * (BM + BN) * STRIDE;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) *reinterpret_cast<uint4*>(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<uint4*>(base + b_lds[i]) = rb[i];
  };

  i32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  const int frag_row = lane & 15, frag_k = (lane >> 4) * 16;
  const int64_t nk = (a.K + BK - 1) / BK;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_tile((kt + 1) * BK);
    const int8_t* base = smem + (kt & 1) * (BM + BN) * STRIDE;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 64) {
      i32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = as_i32x4(*reinterpret_cast<const uint4*>(
            base + (wm * TM + i * 16 + frag_row) * STRIDE + ks + frag_k));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = as_i32x4(*reinterpret_cast<const uint4*>(
            base + BM * STRIDE + (wn * TN + j * 16 + frag_row) * STRIDE + ks + frag_k));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x64(af[i], bf[j], acc[i][j]);
    }
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // ---- fused epilogue
  EpiCol cols[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) cols[j] = load_col(a, n_begin + wn * TN + j * 16 + frag_row, sw, bias);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gr = row_begin + wm * TM + i * 16 + (lane >> 4) * 4 + r;
      EpiRow er;
      er.ok = gr < row_end;
      er.out_row = gr;
      int64_t src = er.ok ? gr : 0;
      if (GROUPED && a.row_ids) {
        src = er.ok ? (int64_t)a.row_ids[gr] : 0;
        if (src < 0 || src >= a.M_src) src = 0;
      }
      er.sx = a.sx_per_token ? a.s_x[src] : a.s_x[0];
      er.zp = (a.azp_mode == 1) ? a.zp[src] : 0;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        epilogue_store(a, er, cols[j], n_begin + wn * TN + j * 16 + frag_row, acc[i][j][r]);
    }
  }
}

namespace {
constexpr int kBM = 128, kBN = 128, kBK = 64;
}

hipError_t launch_scaled_mm(const GemmArgs& a, hipStream_t stream) {
  const int tiles_m = (int)((a.M + kBM - 1) / kBM), tiles_n = (int)((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_i8_kernel<kBM, kBN, kBK, false>), dim3(tiles_m * tiles_n), dim3(256), 0,
                     stream, a, tiles_m, tiles_n);
  return hipGetLastError();
}

const char* scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K) {
  (void)M, (void)N, (void)K;
  return "gemm_i8_kernel<128, 128, 64, false>";
}

hipError_t launch_grouped_mm(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles_m = (a.M + kBM - 1) / kBM + a.E;  // bound on the sum over experts
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_i8_kernel<kBM, kBN, kBK, true>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(256), 0, stream, a, (int)tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace w8a8
