// Prefill-shaped and grouped (MoE) int8 GEMMs on CDNA4 int8 MFMA.
//
// out[t,n] = epilogue( sum_k xq[t,k] * Wq[n,k] ) -- the int8 x int8 -> int32
// product of "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴" (핵심 코드 분석
// §3) against the [out_features, in_features] weight of "vLLM INT8 W8A8 量化实战"
// (4.2), with the scale / zero-point / bias epilogue of the same page (§3-§4)
// fused into the store.
//
// Both operands are K-contiguous ("NT"). A workgroup of 4 waves (2 x 2) owns
// a BM x BN output tile; each wave computes a (BM/2) x (BN/2) sub-tile as a
// grid of 32x32 int32 accumulators with v_mfma_i32_32x32x32_i8 (the form that
// runs at the full int8 rate on gfx950). At 256 x 256 a wave holds 128 x 128
// accumulators (256 AGPRs), so every 16-byte fragment read from LDS feeds
// four MFMAs.
//
// Main kernel (K a multiple of 64): tiles travel HBM -> LDS with the gfx950
// direct-to-LDS load (global_load_lds_dwordx4: each lane's 16 bytes land at
// the wave's LDS base + 16 * lane, no registers involved) into a ring of
// half-stages: half-stage 2s + p holds K step s (BK = 128 or 64 bytes) of the
// A and B rows of tile half p, and the ring fills the LDS (1.5 K steps in
// flight at 256 x 256). One wave instruction fills 64 / (BK / 16) rows of BK
// bytes; the 16-byte chunks of row r sit at a chunk position XOR-swizzled by
// bits of r (swz), which makes the MFMA fragment reads (32 rows x one chunk
// per wave) hit distinct banks whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle. Rows past the end of the matrix load a valid row
// instead; they only feed outputs the epilogue never stores. One barrier per
// K step, before its last k slice, both publishes the next step and retires
// this one, and the instructions are ordered explicitly
// (sched_group_barrier) so that fragment reads and loads slot in between
// MFMAs.
//
// General kernel (any K that is a multiple of 16): the same tile and
// epilogue, with tiles staged through registers (zero-filled past K) into two
// padded LDS buffers.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so the linear
// id is first remapped to give each XCD a contiguous range of tiles, which
// are then walked in groups of 8 tile-rows so that the workgroups running
// together on one XCD share A and B tiles in its L2. The grouped variant maps
// each workgroup to (expert, n-tile, m-tile of that expert's row range), m
// fastest, by scanning expert_offsets (only the first R workgroups have a
// tile, R known on the device; they are the ones remapped across the XCDs);
// rows may be gathered through row_ids.

#include <type_traits>

#include "gemm_common.h"

namespace w8a8 {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Linear workgroup id -> logical tile id such that XCD x (which receives
// workgroups x, x+8, x+16, ...) processes a contiguous range of tiles.
__device__ __forceinline__ int xcd_remap(int pid, int nwg) {
  constexpr int kXcds = 8;
  const int xcd = pid % kXcds, local = pid / kXcds;
  const int base = nwg / kXcds, extra = nwg % kXcds;
  return xcd * base + min(xcd, extra) + local;
}

struct TileLoc {
  int64_t row_begin, row_end;  // output rows [row_begin, min(row_begin + BM, row_end))
  int64_t n_begin;
  int64_t expert;              // -1: no work for this workgroup
};

// Inclusive prefix (sum or maximum) over the 64 lanes of a wave by DPP row
// shifts (1, 2, 4, 8 within each row of 16 lanes) and row broadcasts (lane
// 15 into rows 1 and 3, lane 31 into rows 2 and 3). Lanes with no source take
// the identity 0, so the maximum is over values >= 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <bool MAX>
__device__ __forceinline__ int wave_prefix(int v) {
  auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
  v = op(v, dpp_src<0x111, 0xF>(v));  // row_shr:1
  v = op(v, dpp_src<0x112, 0xF>(v));  // row_shr:2
  v = op(v, dpp_src<0x114, 0xF>(v));  // row_shr:4
  v = op(v, dpp_src<0x118, 0xF>(v));  // row_shr:8
  v = op(v, dpp_src<0x142, 0xA>(v));  // row_bcast:15
  v = op(v, dpp_src<0x143, 0xC>(v));  // row_bcast:31
  return v;
}
__device__ __forceinline__ int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// One block of 64 experts of the grouped tile scan (lane l: expert base + l):
// the clamped segment [s0, s1), its tile count span and the running tile
// count cum (inclusive), continuing from the previous block's carries. Row
// counts fit 32 bits (T < 2^26) and tile counts too (< 2^24, both checked on
// the host).
struct ExpertScan {
  int s0, s1, span, cum;
};
template <int BM>
__device__ __forceinline__ ExpertScan scan_experts(const GemmArgs& a, int64_t base, int carry_s0,
                                                   int carry_cum, int tiles_n) {
  const int T = (int)a.M;
  const int lane = threadIdx.x & 63;
  const int64_t e = base + lane;
  const bool live = e < a.E;
  ExpertScan r;
  const int raw0 = live ? a.expert_offsets[e] : T;
  const int raw1 = live ? a.expert_offsets[e + 1] : T;
  r.s0 = min(max(wave_prefix<true>(max(raw0, 0)), carry_s0), T);
  r.s1 = min(max(raw1, r.s0), T);
  r.span = live ? ((r.s1 - r.s0 + BM - 1) / BM) * tiles_n : 0;
  r.cum = wave_prefix<false>(r.span) + carry_cum;
  return r;
}

template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ TileLoc locate_tile(const GemmArgs& a, int tiles_m, int tiles_n) {
  TileLoc t;
  if (GROUPED) {
    // expert by expert; within an expert, n-tile by n-tile with its m-tiles
    // consecutive, so the workgroups that share a weight tile run together on
    // one XCD and read it from its L2 (an expert's whole weight exceeds it).
    // Every wave scans the experts 64 at a time, one per lane: the clamped
    // segment starts are a running max of the offsets (capped at T), each
    // expert's tile count a running sum, and the expert holding tile `pid` is
    // the lowest lane whose running range contains it.
    // The grid is sized for the most tiles any routing can need; the real
    // count R is known only here. The first R workgroups take the tiles (so
    // every XCD gets an equal share of them: the hardware deals workgroups to
    // the XCDs round-robin), the rest have no work.
    t.n_begin = 0;
    t.expert = -1;
    t.row_begin = t.row_end = 0;
    int total = 0;
    {
      int carry_s0 = 0;
      for (int64_t base = 0; base < a.E; base += 64) {
        const ExpertScan r = scan_experts<BM>(a, base, carry_s0, total, tiles_n);
        carry_s0 = lane_value(r.s0, 63);
        total = lane_value(r.cum, 63);
      }
    }
    if ((int)blockIdx.x >= total) return t;
    const int pid = xcd_remap(blockIdx.x, total);
    const int lane = threadIdx.x & 63;
    int carry_s0 = 0, carry_cum = 0;
    for (int64_t base = 0; base < a.E; base += 64) {
      const ExpertScan r = scan_experts<BM>(a, base, carry_s0, carry_cum, tiles_n);
      const bool live = base + lane < a.E;
      const uint64_t hit = __ballot(live && pid >= r.cum - r.span && pid < r.cum);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        const int e_s0 = lane_value(r.s0, src), e_s1 = lane_value(r.s1, src);
        const int e_first = lane_value(r.cum - r.span, src);
        const int t_e = (e_s1 - e_s0 + BM - 1) / BM;
        const int local = pid - e_first;
        t.expert = base + src;
        t.row_begin = e_s0 + (int64_t)(local % t_e) * BM;
        t.row_end = e_s1;
        t.n_begin = (int64_t)(local / t_e) * BN;
        break;
      }
      carry_s0 = lane_value(r.s0, 63);
      carry_cum = lane_value(r.cum, 63);
    }
  } else {
    const int pid = xcd_remap(blockIdx.x, gridDim.x);
    constexpr int GM = 8;
    const int group = pid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in_group = pid % (GM * tiles_n);
    t.row_begin = (int64_t)(first_m + in_group % gsz) * BM;
    t.row_end = a.M;
    t.n_begin = (int64_t)(in_group / gsz) * BN;
    t.expert = 0;
  }
  return t;
}

// Source row of output row gr (gathered through row_ids in the grouped GEMM),
// or -1 for a row id outside [0, M_src): such a row counts as all zeros. The
// loads then read row 0 instead (a valid address) and the epilogue discards
// the sums.
template <bool GROUPED>
__device__ __forceinline__ int64_t source_row(const GemmArgs& a, int64_t gr) {
  if (GROUPED && a.row_ids) {
    const int64_t s = a.row_ids[gr];
    return (s >= 0 && s < a.M_src) ? s : -1;
  }
  return gr;
}

// The fused epilogue. Its operands are fetched when the workgroup starts
// (epilogue_fetch: thread r takes tile row r and tile column r into
// registers, so the loads' latency hides under the main loop) and published
// to two LDS tables once the main loop is done: per row {all-zero mask,
// token scale, minus the zero point}, per column {weight scale, column sum,
// static correction, bias}. Each wave then turns its sub-tile around one
// 32-row slab at a time: the accumulators go to LDS in MFMA layout (lane =
// column) and come back row-contiguous, each lane taking 8 columns of a row
// (two groups of 4, half the sub-tile apart, so 16 consecutive lanes read
// one contiguous row segment and store whole 128-byte lines).
//
// With one wave per SIMD every VALU instruction costs the wave its full
// issue time, so the per-element work is kept to full-rate instructions:
// the zero-point product uses the 24-bit multiply-add, exact here because a
// zero point fits in 9 bits and a column sum of int8 rows with K <= 65536
// in 24 (|colsum| <= 128 K <= 2^23); row addresses are one per-lane base
// plus a wave-uniform offset. `smem` must hold epilogue_lds_bytes<BM, BN>()
// bytes and be free: the caller has passed a barrier after its last read and
// its last LDS load.
// WM: waves along M (2, or 4 for 8-wave tiles); the waves along N are 2.
template <int BM, int BN, int WM = 2>
constexpr int epilogue_lds_bytes() {
  return 2 * WM * 32 * (BN / 2 + 8) * 4 + BM * 16 + BN * 16;
}

struct EpiFetch {
  int row_mask;    // -1, or 0 for a row that reads as all zeros
  float row_sx;
  int row_zp;
  float col_sw;
  int col_corr;
  uint32_t col_bias;  // bf16 bits
};

template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ EpiFetch epilogue_fetch(const GemmArgs& a, const TileLoc& t,
                                                   const float* sw, const uint16_t* bias) {
  static_assert(BM <= 256 && BN <= 256, "one row and one column per thread");
  EpiFetch f;
  const int r = threadIdx.x;
  const int64_t gr = t.row_begin + (r < BM ? r : 0);
  const int64_t src = gr < t.row_end ? source_row<GROUPED>(a, gr) : -1;
  const int64_t s0 = src > 0 ? src : 0;
  f.row_mask = src >= 0 ? -1 : 0;
  f.row_sx = a.s_x[a.sx_per_token ? s0 : 0];
  // Addresses are selected instead of values (a missing operand reads the
  // scale, which always exists), so the loads carry no use until the epilogue.
  f.row_zp = *(a.azp_mode == 1 ? a.zp + s0 : reinterpret_cast<const int32_t*>(a.s_x));
  const int64_t n = t.n_begin + (r < BN ? r : 0);
  const int64_t nn = n < a.N ? n : 0;
  f.col_sw = sw[a.sw_per_channel ? nn : 0];
  f.col_corr = *(a.azp_mode != 0 ? a.colsum + nn : reinterpret_cast<const int32_t*>(sw));
  f.col_bias = *(bias ? bias + nn : reinterpret_cast<const uint16_t*>(sw));
  return f;
}

// MASKED: rows may read as all zeros (gathered rows). OUT_I32: int32
// output, else bf16. AZP: 0 none, 1 per-token, 2 static, 3 either (read
// from the tables). ST, the store form: per-element stores with row and
// column checks (kStoreScalar); 16-byte (int32) / 8-byte (bf16) stores of
// 4-column groups under a per-row check, when every column of the wave's
// sub-tile is inside the output and ldo allows them (kStoreVecRows: the
// last m-tile of an expert, a ragged M); the same with no check when every
// row is inside too (kStoreVec: the passes then carry no predicate, so the
// compiler is free to run the LDS reads of later passes ahead of earlier
// stores).
enum { kStoreScalar = 0, kStoreVecRows = 1, kStoreVec = 2 };

// FACC: the accumulators hold binary32 bit patterns (the FP8 product), and
// OUT_I32 then means a binary32 output of the scaled value (no AZP).
template <int BM, int BN, bool MASKED, bool OUT_I32, int AZP, int ST, bool FACC = false, int WM = 2>
__device__ __forceinline__ void epilogue_store_tile(const GemmArgs& a, const TileLoc& t, int8_t* smem,
                                                    i32x16 (&acc)[BM / WM / 32][BN / 64]) {
  static_assert(!FACC || AZP == 0, "no zero-point correction on float accumulators");
  constexpr int TM = BM / WM, TN = BN / 2, FM = TM / 32, FN = TN / 32;
  constexpr int CSTRIDE = TN + 8;  // int32 words; rows 4 apart land 32 banks apart
  constexpr int LPR = TN / 8;      // lanes per row
  constexpr int RPP = 64 / LPR >= 8 ? 8 : 4;  // rows per pass
  static_assert(LPR * RPP <= 64 && 32 % RPP == 0, "passes cover the slab");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int frag_row = lane & 31;
  int32_t* slab = reinterpret_cast<int32_t*>(smem) + wave * 32 * CSTRIDE;
  const int4* row_tab = reinterpret_cast<const int4*>(smem + 2 * WM * 32 * CSTRIDE * 4);
  const float* col_sw = reinterpret_cast<const float*>(row_tab + BM);
  const int* col_sum = reinterpret_cast<const int*>(col_sw + BN);
  const int* col_adj = col_sum + BN;
  const float* col_bias = reinterpret_cast<const float*>(col_adj + BN);

  // lanes past whole rows (TN = 96) repeat the first lanes' stores
  const int lw = lane % (LPR * RPP);
  const int q = lw % LPR, lrow = lw / LPR;
  const int cA = 4 * q, cB = TN / 2 + 4 * q;  // the lane's two column groups in the sub-tile
  float sw8[8], bias8[8];
  int sum8[8], adj8[8];
  {
    const int c0 = wn * TN;
    auto get4f = [&](const float* p, float* d) __attribute__((always_inline)) {
      const float4 u = *reinterpret_cast<const float4*>(p + c0 + cA);
      const float4 v = *reinterpret_cast<const float4*>(p + c0 + cB);
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w; d[4] = v.x; d[5] = v.y; d[6] = v.z; d[7] = v.w;
    };
    auto get4i = [&](const int* p, int* d) __attribute__((always_inline)) {
      const int4 u = *reinterpret_cast<const int4*>(p + c0 + cA);
      const int4 v = *reinterpret_cast<const int4*>(p + c0 + cB);
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w; d[4] = v.x; d[5] = v.y; d[6] = v.z; d[7] = v.w;
    };
    if (!OUT_I32 || FACC) get4f(col_sw, sw8), get4f(col_bias, bias8);
    if (AZP == 1 || AZP == 3) get4i(col_sum, sum8);
    if (AZP == 2 || AZP == 3) get4i(col_adj, adj8);
  }
  const int64_t col_a = t.n_begin + wn * TN + cA, col_b = col_a + TN / 2;
  const int lrow0 = wm * TM + lrow;  // the lane's row within the tile, first pass
  using OutT = typename std::conditional<OUT_I32, int32_t, uint16_t>::type;
  OutT* const o_lane = reinterpret_cast<OutT*>(a.out) + (t.row_begin + lrow0) * a.ldo + col_a;

  // Each wave owns its slab and a wave's LDS accesses execute in order, so the
  // slab's writes, its row-contiguous reads and the next slab's writes need no
  // barrier, and the output stores of one slab overlap the next.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        slab[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * CSTRIDE + j * 32 + frag_row] = acc[i][j][r];
#pragma unroll
    for (int p = 0; p < 32 / RPP; ++p) {
      const int lr = p * RPP + lrow;
      const int dr = i * 32 + p * RPP;  // wave-uniform row step from the first pass
      const int4 vA = *reinterpret_cast<const int4*>(slab + lr * CSTRIDE + cA);
      const int4 vB = *reinterpret_cast<const int4*>(slab + lr * CSTRIDE + cB);
      const int4 rp = row_tab[lrow0 + dr];  // {mask, sx, -zp, 0}
      const int v[8] = {vA.x, vA.y, vA.z, vA.w, vB.x, vB.y, vB.z, vB.w};
      int c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        c[k] = MASKED ? v[k] & rp.x : v[k];
        if (AZP == 1 || AZP == 3) c[k] = __mul24(rp.z, sum8[k]) + c[k];
        if (AZP == 2 || AZP == 3) c[k] -= adj8[k];
      }
      OutT* o = o_lane + (int64_t)dr * a.ldo;
      const bool row_ok = ST == kStoreVec || t.row_begin + lrow0 + dr < t.row_end;
      if (OUT_I32 && FACC) {  // the scaled binary32 value, as its bit pattern
        const float sx = __int_as_float(rp.y);
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = __float_as_int(__builtin_fmaf(__int_as_float(c[k]) * sx, sw8[k], bias8[k]));
      }
      if (OUT_I32) {
        if (ST != kStoreScalar) {
          if (row_ok) {
            *reinterpret_cast<int4*>(o) = make_int4(c[0], c[1], c[2], c[3]);
            *reinterpret_cast<int4*>(o + TN / 2) = make_int4(c[4], c[5], c[6], c[7]);
          }
        } else if (row_ok) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((k < 4 ? col_a : col_b) + (k & 3) < a.N) o[(k < 4 ? 0 : TN / 2) + (k & 3)] = c[k];
        }
      } else {
        const float sx = __int_as_float(rp.y);
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const float a0 = FACC ? __int_as_float(c[k]) : (float)c[k];
          const float a1 = FACC ? __int_as_float(c[k + 1]) : (float)c[k + 1];
          const float y0 = __builtin_fmaf(a0 * sx, sw8[k], bias8[k]);
          const float y1 = __builtin_fmaf(a1 * sx, sw8[k + 1], bias8[k + 1]);
          h[k / 2] = pack_bf16x2(y0, y1);
        }
        if (ST != kStoreScalar) {
          if (row_ok) {
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0], h[1]);
            *reinterpret_cast<uint2*>(o + TN / 2) = make_uint2(h[2], h[3]);
          }
        } else if (row_ok) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((k < 4 ? col_a : col_b) + (k & 3) < a.N)
              o[(k < 4 ? 0 : TN / 2) + (k & 3)] = (uint16_t)(h[k / 2] >> (16 * (k & 1)));
        }
      }
    }
  }
}

template <int BM, int BN, bool GROUPED, int ST, bool FACC, int WM = 2>
__device__ __forceinline__ void epilogue_dispatch(const GemmArgs& a, const TileLoc& t, int8_t* smem,
                                                  i32x16 (&acc)[BM / WM / 32][BN / 64]) {
  if constexpr (FACC) {
    if (a.out_i32) epilogue_store_tile<BM, BN, GROUPED, true, 0, ST, true, WM>(a, t, smem, acc);
    else epilogue_store_tile<BM, BN, GROUPED, false, 0, ST, true, WM>(a, t, smem, acc);
  } else if (a.out_i32) {
    if (a.azp_mode == 1) epilogue_store_tile<BM, BN, GROUPED, true, 1, ST, false, WM>(a, t, smem, acc);
    else if (a.azp_mode == 2) epilogue_store_tile<BM, BN, GROUPED, true, 2, ST, false, WM>(a, t, smem, acc);
    else epilogue_store_tile<BM, BN, GROUPED, true, 0, ST, false, WM>(a, t, smem, acc);
  } else {
    if (a.azp_mode == 1) epilogue_store_tile<BM, BN, GROUPED, false, 1, ST, false, WM>(a, t, smem, acc);
    else if (a.azp_mode == 2) epilogue_store_tile<BM, BN, GROUPED, false, 2, ST, false, WM>(a, t, smem, acc);
    else epilogue_store_tile<BM, BN, GROUPED, false, 0, ST, false, WM>(a, t, smem, acc);
  }
}

template <int BM, int BN, bool GROUPED, bool FACC = false, int WM = 2>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const TileLoc& t, const EpiFetch& f,
                                              int8_t* smem, i32x16 (&acc)[BM / WM / 32][BN / 64]) {
  static_assert(WM == 2 || FACC, "the integer forms run on 4-wave tiles");
  constexpr int TN = BN / 2;
  constexpr int CSTRIDE = TN + 8;
  int4* row_tab = reinterpret_cast<int4*>(smem + 2 * WM * 32 * CSTRIDE * 4);
  float* col_sw = reinterpret_cast<float*>(row_tab + BM);
  int* col_sum = reinterpret_cast<int*>(col_sw + BN);
  int* col_adj = col_sum + BN;
  float* col_bias = reinterpret_cast<float*>(col_adj + BN);
  const int r = threadIdx.x;
  if (r < BM) row_tab[r] = make_int4(f.row_mask, __float_as_int(f.row_sx), a.azp_mode == 1 ? -f.row_zp : 0, 0);
  if (r < BN) {
    col_sw[r] = f.col_sw;
    col_sum[r] = a.azp_mode == 1 ? f.col_corr : 0;
    col_adj[r] = a.azp_mode == 2 ? f.col_corr : 0;
    col_bias[r] = a.bias ? __uint_as_float(f.col_bias << 16) : 0.0f;
  }
  // the tables are visible to every wave; no wait for global stores
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int wn = (threadIdx.x >> 6) & 1;
  // groups of 4 columns leave as 16-byte (int32) or 8-byte (bf16) stores when
  // the wave's columns are all inside the output; rows past the tile's end
  // (the last m-tile of an expert, a ragged M) only switch those stores off
  const bool vec = t.n_begin + (wn + 1) * TN <= a.N && a.ldo % 4 == 0;
  const bool rows = t.row_begin + BM <= t.row_end;
  if (!vec) {
    if constexpr (FACC) {
      if (a.out_i32) epilogue_store_tile<BM, BN, GROUPED, true, 0, kStoreScalar, true, WM>(a, t, smem, acc);
      else epilogue_store_tile<BM, BN, GROUPED, false, 0, kStoreScalar, true, WM>(a, t, smem, acc);
    } else if (a.out_i32) {
      epilogue_store_tile<BM, BN, GROUPED, true, 3, kStoreScalar, false, WM>(a, t, smem, acc);
    } else {
      epilogue_store_tile<BM, BN, GROUPED, false, 3, kStoreScalar, false, WM>(a, t, smem, acc);
    }
  } else if (rows) {
    epilogue_dispatch<BM, BN, GROUPED, kStoreVec, FACC, WM>(a, t, smem, acc);
  } else {
    epilogue_dispatch<BM, BN, GROUPED, kStoreVecRows, FACC, WM>(a, t, smem, acc);
  }
}

// Workgroup barrier without the memory fence __syncthreads() carries (which
// would wait for every load in flight, including the prefetched stages). The
// ordering the direct-to-LDS ring needs is explicit: each wave waits for its
// own loads of the stage with s_waitcnt vmcnt before the barrier, and the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { __asm__ volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- main kernel
// Chunk position of logical 16-byte chunk c in tile row r (CH chunks per
// row): distinct banks for the fragment reads of 8 consecutive rows (32-bank
// view) and of 16 consecutive rows (64-bank view). Depends on bits 0-4 of r
// only, so rows 32 apart (the MFMA blocks of one wave) share it.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  return CH == 4 ? (((r >> 1) ^ (r >> 3)) & 3) : ((r ^ ((r >> 3) & 3)) & 7);
}

// The ring kernel's body, for int8 operands (v_mfma_i32_32x32x32_i8, exact
// int32 sums) or, with FP8, for E4M3 operands (v_mfma_scale_f32_32x32x64_f8f6f4
// with unit block scales: 64 k per instruction from two 16-byte fragment
// reads per lane, binary32 sums kept as bit patterns in the same registers).
template <int BM, int BN, int BK, int NH, bool GROUPED, bool FP8>
__device__ __forceinline__ void gemm_dma_body(const GemmArgs& a, int tiles_m, int tiles_n) {
  constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
  // The ring is made of NH half-stages: half-stage 2s + p holds K step s of
  // the A rows [p*TM, p*TM + TM) and the B rows [p*TN, p*TN + TN) -- the
  // operands of the waves in tile row p and tile column p.
  constexpr int HSTAGE = (TM + TN) * BK;
  constexpr int CH = BK / 16;                 // 16-byte chunks per tile row
  constexpr int RPI = 64 / CH;                // tile rows per 1-KiB load instruction
  constexpr int AI = TM / RPI / 4, BI = TN / RPI / 4;  // load instructions per wave per half-stage
  constexpr int PER_HALF = AI + BI;
  constexpr int KS = BK / (FP8 ? 64 : 32);    // MFMA k slices per K step
  constexpr int RPF = FP8 ? 2 : 1;            // 16-byte LDS reads per fragment
  static_assert(CH == 4 || CH == 8, "BK is 64 or 128");
  static_assert(TM % (4 * RPI) == 0 && TN % (4 * RPI) == 0, "tile / load mismatch");
  static_assert(NH >= 5 && (NH - 3) * PER_HALF <= 63, "ring / vmcnt range");
  static_assert(epilogue_lds_bytes<BM, BN>() <= NH * HSTAGE, "epilogue does not fit the LDS");

  __shared__ __attribute__((aligned(1024))) int8_t smem[NH * HSTAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileLoc t = locate_tile<BM, BN, GROUPED>(a, tiles_m, tiles_n);
  if (t.expert < 0) return;
  const int8_t* B = a.B + t.expert * a.N * a.ldb;
  const float* sw = a.s_w + (GROUPED ? t.expert * a.N : 0);
  const uint16_t* bias = (GROUPED && a.bias) ? a.bias + t.expert * a.N : a.bias;
  // issued before the ring's loads, so the ring's vmcnt waits retire them too
  const EpiFetch ef = epilogue_fetch<BM, BN, GROUPED>(a, t, sw, bias);

  // ---- per-lane DMA sources: in half-stage part p, instruction q of this
  // wave fills tile rows p*TM + (wave*AI + q)*RPI .. +RPI-1 of A (likewise
  // for B); lane l writes row +l/CH, physical chunk l%CH, which holds logical
  // chunk (l%CH) ^ swz(row).
  const int lrow = lane / CH, pch = lane % CH;
  const int8_t* a_src[2][AI];
  const int8_t* b_src[2][BI];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int q = 0; q < AI; ++q) {
      const int r = p * TM + (wave * AI + q) * RPI + lrow;
      const int64_t gr = min(t.row_begin + r, t.row_end - 1);
      const int64_t src = source_row<GROUPED>(a, gr);
      a_src[p][q] = a.A + (src > 0 ? src : 0) * a.lda + (pch ^ swz<CH>(r)) * 16;
    }
#pragma unroll
    for (int q = 0; q < BI; ++q) {
      const int r = p * TN + (wave * BI + q) * RPI + lrow;
      const int64_t n = min(t.n_begin + r, a.N - 1);
      b_src[p][q] = B + n * a.ldb + (pch ^ swz<CH>(r)) * 16;
    }
  }
  const int nk = (int)(a.K / BK);
  // Load instruction q (of PER_HALF) of half-stage h: K step h / 2 (past the
  // last K step it reloads the last one), part P = h % 2, into ring slot
  // h % NH. P is known where it is called, so the source pointers are picked
  // at compile time.
  auto issue_one = [&](int h, auto part, int q) __attribute__((always_inline)) {
    constexpr int P = decltype(part)::value;
    int8_t* dst = smem + (h % NH) * HSTAGE;
    const int64_t k0 = (int64_t)min(h >> 1, nk - 1) * BK;
    if (q < AI)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(a_src[P][q] + k0),
                                       (lds_void_ptr)(dst + (wave * AI + q) * 1024), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((global_void_ptr)(b_src[P][q - AI] + k0),
                                       (lds_void_ptr)(dst + TM * BK + (wave * BI + q - AI) * 1024), 16,
                                       0, 0);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using PA = std::integral_constant<int, (NH - 1) & 1>;  // part of the half-stage issued in region A
  using PB = std::integral_constant<int, NH & 1>;        // part of the half-stage issued in region B

  // ---- fragment reads of K step s: lane reads tile row (.. + lane%32),
  // logical chunk 2*ks + lane/32 of the BK-byte row, from the half-stage of
  // this wave's tile row (A) and tile column (B); rows 32 apart share swz().
  const int fr = lane & 31;
  const int fsw = swz<CH>(fr);
  using Frag = typename std::conditional<FP8, i32x8, i32x4>::type;
  Frag fa[2][FM], fb[2][FN];
  // int8: the lane's 16 bytes of the 32-deep slice; FP8: its 32 bytes of the
  // 64-deep slice (two chunks), the same k positions in A and in B
  auto frag_at = [&](const int8_t* p, int ks) __attribute__((always_inline)) -> Frag {
    if constexpr (FP8) {
      const int c0 = 4 * ks + 2 * (lane >> 5);
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p + ((c0 ^ fsw) * 16));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + (((c0 + 1) ^ fsw) * 16));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const i32x4*>(p + (((2 * ks + (lane >> 5)) ^ fsw) * 16));
    }
  };
  auto read_one = [&](int s, int ks, int slot, int f) __attribute__((always_inline)) {
    if (f < FM) {
      const int8_t* sa = smem + ((2 * s + wm) % NH) * HSTAGE + fr * BK;
      fa[slot][f] = frag_at(sa + f * 32 * BK, ks);
    } else {
      const int8_t* sb = smem + ((2 * s + wn) % NH) * HSTAGE + TM * BK + fr * BK;
      fb[slot][f - FM] = frag_at(sb + (f - FM) * 32 * BK, ks);
    }
  };

  i32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (FP8) acc[i][j] = mfma32x32x64_fp8(fa[slot][i], fb[slot][j], acc[i][j]);
        else acc[i][j] = mfma32x32x32(fa[slot][i], fb[slot][j], acc[i][j]);
      }
  };
  static_assert(KS % 2 == 0, "the next step's first slice reuses fragment slot 0");
  constexpr int NR = FM + FN, NM = FM * FN;
  static_assert(NM >= NR, "more fragment reads than MFMAs in a slice");
  // Region A's loads go out one after every RA-th fragment read.
  constexpr int READS_A = (KS - 1) * NR;
  constexpr int RA = READS_A / PER_HALF;
  static_assert(RA >= 1, "region A has fewer fragment reads than loads");

  // Half-stages 0 .. NH-2 are requested up front. Step kt then requests two
  // more, each into the slot of a retired half-stage: half-stage 2kt + NH - 1
  // (the second half of step kt-1's slots, retired at the previous barrier)
  // spread over the step's first slices, and half-stage 2kt + NH (the first
  // of step kt's own slots) right after the barrier. The loads in flight
  // reach one and a half K steps ahead, each barrier waits only for the
  // half-stage requested in the step before, and no slice issues more than
  // a few loads: a load instruction that has to wait for the memory pipeline
  // holds up the MFMAs queued behind it in the same wave. Past the last K
  // step the requests reload it into retired slots (same addresses, never
  // read), which keeps every step one straight-line block.
#pragma unroll
  for (int h = 0; h < NH - 1; ++h)
#pragma unroll
    for (int q = 0; q < PER_HALF; ++q) {
      if (h % 2 == 0) issue_one(h, P0{}, q);
      else issue_one(h, P1{}, q);
    }
  wait_vmcnt<(NH - 3) * PER_HALF>();
  barrier_no_fence();  // every wave's part of K step 0 has landed
#pragma unroll
  for (int f = 0; f < NR; ++f) read_one(0, 0, 0, f);

  for (int kt = 0; kt < nk; ++kt) {
    // Region A, all slices but the last: each slice's MFMAs with the next
    // slice's fragment reads slotted in after the first of them, and one
    // load of half-stage 2kt + NH - 1 after every RA-th read.
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) {
#pragma unroll
      for (int f = 0; f < NR; ++f) {
        read_one(kt, s + 1, (s + 1) & 1, f);
        const int r = s * NR + f;
        if (r % RA == RA - 1 && r / RA < PER_HALF) issue_one(2 * kt + NH - 1, PA{}, r / RA);
      }
      mfmas(s & 1);
    }
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < NR) {
          __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
          const int r = s * NR + q;
          if (r % RA == RA - 1 && r / RA < PER_HALF) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
      }
    }
    // Before the last slice (its fragments are already in registers): this
    // wave's parts of K step kt+1 have landed once the NH - 4 half-stages
    // requested after them are all that is outstanding, and its reads of K
    // step kt are done. After the barrier every wave's parts of step kt+1 are
    // visible and no wave reads step kt again, so its slots take the next
    // requests and the first fragments of step kt+1 are read under the last
    // slice's MFMAs: no step starts by waiting for LDS.
    __builtin_amdgcn_sched_barrier(0);  // MFMAs do not cross the wait either
    wait_vmcnt<(NH - 4) * PER_HALF>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // Region B, the last slice: the next step's first fragment reads, each
    // followed by one load of half-stage 2kt + NH.
#pragma unroll
    for (int f = 0; f < NR; ++f) {
      read_one(kt + 1, 0, 0, f);
      if (f < PER_HALF) issue_one(2 * kt + NH, PB{}, f);
    }
#pragma unroll
    for (int q = NR; q < PER_HALF; ++q) issue_one(2 * kt + NH, PB{}, q);
    mfmas((KS - 1) & 1);
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < NR) {
        __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
        if (q < PER_HALF) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      } else if (q < PER_HALF) {
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      }
    }
  }
  __syncthreads();  // waits for every load, including the reloads past the last step
  epilogue_tile<BM, BN, GROUPED, FP8>(a, t, ef, smem, acc);
}

template <int BM, int BN, int BK, int NH, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_i8_dma_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  gemm_dma_body<BM, BN, BK, NH, GROUPED, false>(a, tiles_m, tiles_n);
}

// The W8A8 FP8 product with a per-tensor / per-channel weight scale and a
// per-token / per-tensor activation scale, applied in the epilogue.
template <int BM, int BN, int NH>
__global__ __launch_bounds__(256) void gemm_fp8_dma_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  gemm_dma_body<BM, BN, 128, NH, false, true>(a, tiles_m, tiles_n);
}

// ------------------------------------------------------------- general kernel
template <int BM, int BN, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_i8_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int NT = 256, BK = 64;
  constexpr int STRIDE = BK + 16;
  constexpr int STAGE = (BM + BN) * STRIDE;
  constexpr int TM = BM / 2, TN = BN / 2;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int KC = BK / 16;
  constexpr int A_PER_T = BM * KC / NT, B_PER_T = BN * KC / NT;
  static_assert(BM * KC % NT == 0 && BN * KC % NT == 0, "tile / thread mismatch");
  static_assert(epilogue_lds_bytes<BM, BN>() <= 2 * STAGE, "epilogue does not fit the LDS");

  __shared__ __attribute__((aligned(16))) int8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileLoc t = locate_tile<BM, BN, GROUPED>(a, tiles_m, tiles_n);
  if (t.expert < 0) return;
  const int8_t* B = a.B + t.expert * a.N * a.ldb;
  const float* sw = a.s_w + (GROUPED ? t.expert * a.N : 0);
  const uint16_t* bias = (GROUPED && a.bias) ? a.bias + t.expert * a.N : a.bias;
  const EpiFetch ef = epilogue_fetch<BM, BN, GROUPED>(a, t, sw, bias);

  // ---- per-thread global source pointers (fixed over K)
  const int8_t* a_src[A_PER_T];
  bool a_ok[A_PER_T];
  int a_kc[A_PER_T], a_lds[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = tid + i * NT, r = c / KC, kc = c % KC;
    const int64_t gr = t.row_begin + r;
    const int64_t src = gr < t.row_end ? source_row<GROUPED>(a, gr) : -1;
    a_ok[i] = src >= 0;
    a_src[i] = a.A + (a_ok[i] ? src : 0) * a.lda + kc * 16;
    a_kc[i] = kc * 16;
    a_lds[i] = r * STRIDE + kc * 16;
  }
  const int8_t* b_src[B_PER_T];
  bool b_ok[B_PER_T];
  int b_kc[B_PER_T], b_lds[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int c = tid + i * NT, r = c / KC, kc = c % KC;
    const int64_t n = t.n_begin + r;
    b_ok[i] = n < a.N;
    b_src[i] = B + (b_ok[i] ? n : 0) * a.ldb + kc * 16;
    b_kc[i] = kc * 16;
    b_lds[i] = BM * STRIDE + r * STRIDE + kc * 16;
  }

  // Loads are branch-free: an out-of-range chunk reads a valid address and is
  // replaced by zeros (the K tail must be zero in both operands).
  u32x4 ra[A_PER_T], rb[B_PER_T];
  auto load_tile = [&](int64_t k0) __attribute__((always_inline)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const bool ok = a_ok[i] && k0 + a_kc[i] < a.K;
      const u32x4 v = *reinterpret_cast<const u32x4*>(a_src[i] + (ok ? k0 : 0));
      ra[i] = ok ? v : z;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const bool ok = b_ok[i] && k0 + b_kc[i] < a.K;
      const u32x4 v = *reinterpret_cast<const u32x4*>(b_src[i] + (ok ? k0 : 0));
      rb[i] = ok ? v : z;
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    int8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) *reinterpret_cast<u32x4*>(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<u32x4*>(base + b_lds[i]) = rb[i];
  };

  i32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int frag_row = lane & 31, frag_k = (lane >> 5) * 16;
  const int a_frag = (wm * TM + frag_row) * STRIDE + frag_k;
  const int b_frag = BM * STRIDE + (wn * TN + frag_row) * STRIDE + frag_k;
  const int64_t nk = (a.K + BK - 1) / BK;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_tile((kt + 1) * BK);
    const int8_t* base = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      i32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(base + a_frag + i * 32 * STRIDE + ks);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(base + b_frag + j * 32 * STRIDE + ks);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x32(af[i], bf[j], acc[i][j]);
    }
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
  }
  epilogue_tile<BM, BN, GROUPED>(a, t, ef, smem, acc);
}

// ------------------------------------------------------------- FP8 kernel
// The W8A8 FP8 product for the 128 x 128 block scales of "[SGLang] W4A8,
// W8A8, W4A4: 혼합 정밀도 양자화 스킴" (핵심 코드 분석 §1-§2, the block path),
// and for per-tensor / per-channel scales when K is not a multiple of 128.
// Tiles are staged through registers into two LDS buffers (XOR-swizzled as
// in the ring kernel), one 128-deep K step (one scale block) per buffer, zero
// codes past K. With BLOCK, each K step's sums go to a fresh set of
// accumulators, which are then scaled by s_x[g, t] * s_w[n / 128, g] and
// added into the running ones (the block scales are applied per K block, so
// they cannot wait for the epilogue); the epilogue then adds only the bias.
// Activation scales are group-major [G, M], weight scales [ceil(N/128), G].
template <int BM, int BN, bool BLOCK>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int NT = 256, BK = 128, CH = BK / 16;
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int SXB = BLOCK ? BM * 4 : 0;  // the step's activation scales after the tiles
  constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
  constexpr int A_PER_T = BM * CH / NT, B_PER_T = BN * CH / NT;
  static_assert(BM * CH % NT == 0 && BN * CH % NT == 0, "tile / thread mismatch");
  static_assert(!BLOCK || (BN == 128 && BM <= NT), "a block-scaled tile spans one 128-column weight block");
  static_assert(epilogue_lds_bytes<BM, BN>() <= 2 * (STAGE + SXB), "epilogue does not fit the LDS");

  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * (STAGE + SXB)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TileLoc t = locate_tile<BM, BN, false>(a, tiles_m, tiles_n);
  const float* sw = a.s_w;
  EpiFetch ef = epilogue_fetch<BM, BN, false>(a, t, sw, a.bias);
  if (BLOCK) {  // the scales are applied in the main loop
    ef.row_sx = 1.0f;
    ef.col_sw = 1.0f;
  }

  // per-thread chunks: chunk c = tid + i * NT of the A (B) tile is row c / CH,
  // logical chunk c % CH, stored at chunk position (c % CH) ^ swz(row)
  const int8_t* a_src[A_PER_T];
  int a_lds[A_PER_T], a_kc[A_PER_T];
  bool a_ok[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = tid + i * NT, r = c / CH, kc = c % CH;
    const int64_t gr = t.row_begin + r;
    a_ok[i] = gr < t.row_end;
    a_src[i] = a.A + (a_ok[i] ? gr : 0) * a.lda + kc * 16;
    a_kc[i] = kc * 16;
    a_lds[i] = r * BK + ((kc ^ swz<CH>(r)) * 16);
  }
  const int8_t* b_src[B_PER_T];
  int b_lds[B_PER_T], b_kc[B_PER_T];
  bool b_ok[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int c = tid + i * NT, r = c / CH, kc = c % CH;
    const int64_t n = t.n_begin + r;
    b_ok[i] = n < a.N;
    b_src[i] = a.B + (b_ok[i] ? n : 0) * a.ldb + kc * 16;
    b_kc[i] = kc * 16;
    b_lds[i] = BM * BK + r * BK + ((kc ^ swz<CH>(r)) * 16);
  }
  const int64_t G = (a.K + BK - 1) / BK;
  const int64_t sx_row = min(t.row_begin + (tid < BM ? tid : 0), a.M - 1);
  const int64_t nb = t.n_begin / 128;

  u32x4 ra[A_PER_T], rb[B_PER_T];
  float rs = 0.0f;
  auto load_tile = [&](int64_t g) __attribute__((always_inline)) {
    const int64_t k0 = g * BK;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const bool ok = a_ok[i] && k0 + a_kc[i] < a.K;
      const u32x4 v = *reinterpret_cast<const u32x4*>(a_src[i] + (ok ? k0 : 0));
      ra[i] = ok ? v : z;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const bool ok = b_ok[i] && k0 + b_kc[i] < a.K;
      const u32x4 v = *reinterpret_cast<const u32x4*>(b_src[i] + (ok ? k0 : 0));
      rb[i] = ok ? v : z;
    }
    if (BLOCK) rs = a.s_x[g * a.M + sx_row];
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    int8_t* base = smem + buf * (STAGE + SXB);
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) *reinterpret_cast<u32x4*>(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<u32x4*>(base + b_lds[i]) = rb[i];
    if (BLOCK && tid < BM) reinterpret_cast<float*>(base + STAGE)[tid] = rs;
  };

  i32x16 acc[FM][FN], part[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int fr = lane & 31, fsw = swz<CH>(fr);
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int64_t g = 0; g < G; ++g) {
    const bool more = g + 1 < G;
    if (more) load_tile(g + 1);
    const int8_t* base = smem + (g & 1) * (STAGE + SXB);
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      const int c0 = 4 * ks + 2 * (lane >> 5);
      i32x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int8_t* p = base + (wm * TM + 32 * i + fr) * BK;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(p + ((c0 ^ fsw) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(p + (((c0 + 1) ^ fsw) * 16));
        af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int8_t* p = base + BM * BK + (wn * TN + 32 * j + fr) * BK;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(p + ((c0 ^ fsw) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(p + (((c0 + 1) ^ fsw) * 16));
        bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (BLOCK) {
            i32x16 z = {};
            part[i][j] = mfma32x32x64_fp8(af[i], bf[j], ks == 0 ? z : part[i][j]);
          } else {
            acc[i][j] = mfma32x32x64_fp8(af[i], bf[j], acc[i][j]);
          }
        }
    }
    if (BLOCK) {
      // acc += part * s_x[g, row] * s_w[nb, g]; the lane's rows of fragment i
      // are 32 i + 8 q + 4 (lane / 32) + (0..3), q = register / 4
      const float swg = sw[nb * G + g];
      const float* sx = reinterpret_cast<const float*>(base + STAGE) + wm * TM + 4 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 s4 = *reinterpret_cast<const float4*>(sx + 32 * i + 8 * q);
          const float sc[4] = {s4.x * swg, s4.y * swg, s4.z * swg, s4.w * swg};
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][4 * q + r] = __float_as_int(__builtin_fmaf(__int_as_float(part[i][j][4 * q + r]), sc[r],
                                                                   __int_as_float(acc[i][j][4 * q + r])));
        }
    }
    if (more) store_tile((g + 1) & 1);
    __syncthreads();
  }
  epilogue_tile<BM, BN, false, true>(a, t, ef, smem, acc);
}

// The block-scaled FP8 product on BM x 128 tiles (BM = 128 with 4 waves, or
// 256 with 8) with its operands in a ring of S direct-to-LDS stages (K a
// multiple of 128): stage g holds K step g (one scale block) of the tile's
// BM A rows and 128 B rows (XOR-swizzled 16-byte chunks, as in the ring
// kernel), the step's BM activation scales and its weight-block scale. Every
// wave owns a 64 x 64 sub-tile and issues the same loads per stage (4 of A,
// 16 / NW of B, one of 32 activation scales plus a copy of the weight scale),
// so its own vmcnt tells it when its part of a stage has landed, and no other
// global load sits behind them in the loop. S - 1 stages are in flight;
// stage g + S - 1 goes into the slot step g - 1 used, after the barrier that
// opens step g. Each step's two 64-deep slices go to fresh accumulators,
// which are scaled by s_x[g, row] * s_w[n / 128, g] and added into the
// running ones. That scaling is VALU work the MFMA pipe cannot hide within
// one wave, so every SIMD runs two waves: two 4-wave workgroups per CU with
// S = 2 (66 KiB of LDS each), or one 8-wave workgroup.
template <int S, int BM>
__global__ __launch_bounds__(BM * 2) void gemm_fp8_block_dma_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int BN = 128, BK = 128, CH = BK / 16;
  constexpr int NW = BM / 32, WM = NW / 2;  // waves; waves along M (2 along N)
  constexpr int FM = 2, FN = 2;             // 32 x 32 fragments of a wave's 64 x 64 sub-tile
  constexpr int BQ = 16 / NW;               // B load instructions per wave and stage
  constexpr int AB = (BM + BN) * BK;        // tile bytes of a stage
  constexpr int SCB = (NW * 256 + 1023) / 1024 * 1024;  // NW x 256 B of scales (wave w: s_x rows 32w.., then s_w)
  constexpr int STG = AB + SCB;
  constexpr int PER_STAGE = 4 + BQ + 1;     // loads per wave per stage
  static_assert(BM == 128 || BM == 256, "4 or 8 waves");
  static_assert(S >= 2 && (S - 2) * PER_STAGE <= 63, "ring / vmcnt range");
  static_assert(epilogue_lds_bytes<BM, BN, WM>() <= S * STG, "epilogue does not fit the LDS");
  static_assert(S * STG <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) int8_t smem[S * STG];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TileLoc t = locate_tile<BM, BN, false>(a, tiles_m, tiles_n);
  EpiFetch ef = epilogue_fetch<BM, BN, false>(a, t, a.s_w, a.bias);
  ef.row_sx = 1.0f;  // the scales are applied in the main loop
  ef.col_sw = 1.0f;
  const int G = (int)(a.K / BK);
  const int64_t nb = t.n_begin / 128;

  // DMA sources: A instruction q of this wave fills tile rows (wave * 4 + q) * 8
  // .. + 7, B instruction q rows (wave * BQ + q) * 8 .. + 7; lane l writes row
  // + l / 8, physical chunk l % 8, which holds logical chunk (l % 8) ^ swz(row).
  // Rows past the matrix load its last row (never stored).
  const int lrow = lane >> 3, pch = lane & 7;
  const int8_t* a_src[4];
  const int8_t* b_src[BQ];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (wave * 4 + q) * 8 + lrow;
    a_src[q] = a.A + min(t.row_begin + r, a.M - 1) * a.lda + ((pch ^ swz<CH>(r)) * 16);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int r = (wave * BQ + q) * 8 + lrow;
    b_src[q] = a.B + min(t.n_begin + r, a.N - 1) * a.ldb + ((pch ^ swz<CH>(r)) * 16);
  }
  // scales: lanes 0 .. 31 of wave w load s_x of rows 32 w .. 32 w + 31,
  // lane 32 the weight block's scale (group-major s_x, stride M; s_w stride 1)
  const bool sc_lane = lane <= 32;
  const float* sc_src = lane < 32 ? a.s_x + min(t.row_begin + wave * 32 + lane, a.M - 1) : a.s_w + nb * G;
  const int64_t sc_step = lane < 32 ? a.M : 1;

  // the loads of stage h into slot h % S (past the last step: a reload of it)
  auto issue = [&](int h) __attribute__((always_inline)) {
    int8_t* dst = smem + (h % S) * STG;
    const int g = min(h, G - 1);
    const int64_t k0 = (int64_t)g * BK;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(a_src[q] + k0), (lds_void_ptr)(dst + (wave * 4 + q) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int q = 0; q < BQ; ++q)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(b_src[q] + k0),
                                       (lds_void_ptr)(dst + BM * BK + (wave * BQ + q) * 1024), 16, 0, 0);
    if (sc_lane)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(sc_src + g * sc_step), (lds_void_ptr)(dst + AB + wave * 256),
                                       4, 0, 0);
  };

  i32x16 acc[FM][FN], part[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int fr = lane & 31, fsw = swz<CH>(fr);
#pragma unroll
  for (int h = 0; h < S - 1; ++h) issue(h);
  for (int g = 0; g < G; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(S - 2) * PER_STAGE>();  // this wave's part of stage g has landed
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(g + S - 1);  // into the slot of step g - 1, which every wave has finished reading
    const int8_t* base = smem + (g % S) * STG;
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      const int c0 = 4 * ks + 2 * (lane >> 5);
      i32x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int8_t* p = base + (wm * 64 + 32 * i + fr) * BK;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(p + ((c0 ^ fsw) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(p + (((c0 + 1) ^ fsw) * 16));
        af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int8_t* p = base + BM * BK + (wn * 64 + 32 * j + fr) * BK;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(p + ((c0 ^ fsw) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(p + (((c0 + 1) ^ fsw) * 16));
        bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          i32x16 z = {};
          part[i][j] = mfma32x32x64_fp8(af[i], bf[j], ks == 0 ? z : part[i][j]);
        }
    }
    // acc += part * s_x[g, row] * s_w[nb, g]; the lane's rows of fragment i
    // are 32 i + 8 q + 4 (lane / 32) + (0..3), q = register / 4. The scales
    // are read as integers, like the tiles: typed float reads of the stage
    // make the compiler wait for every load in flight.
    const int* scl = reinterpret_cast<const int*>(base + AB);
    const float swg = __int_as_float(scl[wave * 64 + 32]);
    const int* sx = scl + wm * 128 + 4 * (lane >> 5);  // s_x of row 32 b + r sits at 64 b + r
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x4 s4 = *reinterpret_cast<const i32x4*>(sx + 64 * i + 8 * q);  // rows 32 (2 wm + i) + ..
        const float sc[4] = {__int_as_float(s4[0]) * swg, __int_as_float(s4[1]) * swg, __int_as_float(s4[2]) * swg,
                             __int_as_float(s4[3]) * swg};
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][4 * q + r] = __float_as_int(__builtin_fmaf(__int_as_float(part[i][j][4 * q + r]), sc[r],
                                                                 __int_as_float(acc[i][j][4 * q + r])));
      }
  }
  wait_vmcnt<0>();
  __syncthreads();  // every load has landed, including the reloads past the last step
  epilogue_tile<BM, BN, false, true, WM>(a, t, ef, smem, acc);
}

namespace {

struct TileCfg {
  int bm, bn;
};

// Tile menu: 256 x 256 (each LDS fragment feeds 4 MFMAs) when the problem has
// enough tiles to fill the 256 compute units, 256 x 192 / 256 x 128 /
// 128 x 128 when the big tile would leave much of the chip idle (2048 x 6144
// makes 192 tiles of 256 x 256 but exactly 256 of 256 x 192). Estimated cost
// = rounds of workgroups over the CUs x tile area / measured relative
// throughput per unit of tile area (1.0, 0.82, 0.81, 0.72 for the four sizes
// on 8192 x 4096 x 4096 with BK = 128).
// K-step variant: 128-byte steps (full cache lines per row and load) when K
// allows, 64-byte steps otherwise, registers-staged with zero fill for any
// other K.
enum KVariant { kK128 = 0, kK64 = 1, kKAny = 2 };
KVariant pick_k(int64_t K) { return K % 128 == 0 ? kK128 : (K % 64 == 0 ? kK64 : kKAny); }

TileCfg pick_tile(int64_t M, int64_t N, int64_t K) {
  const TileCfg menu[4] = {{256, 256}, {256, 192}, {256, 128}, {128, 128}};
  const double eff[4] = {1.0, 0.82, 0.81, 0.72};
  int best = 0;
  double best_cost = 0;
  for (int c = 0; c < 4; ++c) {
    if (menu[c].bn == 192 && pick_k(K) == kK64) continue;  // 96-column halves need 128-byte steps
    const int64_t tiles = ((M + menu[c].bm - 1) / menu[c].bm) * ((N + menu[c].bn - 1) / menu[c].bn);
    const int64_t rounds = (tiles + 255) / 256;
    const double cost = (double)rounds * menu[c].bm * menu[c].bn / eff[c];
    if (c == 0 || cost < best_cost) {
      best = c;
      best_cost = cost;
    }
  }
  return menu[best];
}

// The ring takes as many half-stages (up to 10) as the 160 KiB of LDS hold.

template <int BM, int BN, int BK>
constexpr int ring_halves() {
  constexpr int kLds = 160 * 1024;
  constexpr int n = kLds / ((BM + BN) / 2 * BK);
  return n < 10 ? n : 10;
}
static_assert(ring_halves<256, 256, 128>() == 5 && ring_halves<256, 192, 128>() == 5 &&
                  ring_halves<256, 128, 128>() == 6 && ring_halves<128, 128, 128>() == 10 &&
                  ring_halves<256, 256, 64>() == 10 && ring_halves<256, 128, 64>() == 10 &&
                  ring_halves<128, 128, 64>() == 10,
              "ring sizes the kernel names below state");

template <int BM, int BN, bool GROUPED>
hipError_t launch_tiles(const GemmArgs& a, int64_t extra_m_tiles, hipStream_t stream) {
  const int64_t tiles_m = (a.M + BM - 1) / BM + extra_m_tiles;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
  KVariant kv = pick_k(a.K);
  if (kv == kK64 && BN == 192) kv = kKAny;  // not picked (pick_tile); kept launchable
  switch (kv) {
    case kK128:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<BM, BN, 128, ring_halves<BM, BN, 128>(), GROUPED>), grid,
                         block, 0, stream, a, (int)tiles_m, tiles_n);
      break;
    case kK64:
      if constexpr (BN != 192)
        hipLaunchKernelGGL((gemm_i8_dma_kernel<BM, BN, 64, ring_halves<BM, BN, 64>(), GROUPED>), grid,
                           block, 0, stream, a, (int)tiles_m, tiles_n);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, GROUPED>), grid, block, 0, stream, a, (int)tiles_m,
                         tiles_n);
  }
  return hipGetLastError();
}

const char* kernel_name(int bm, int bn, bool grouped, int64_t K) {
  static const char* names[3][2][4] = {
      {{"gemm_i8_dma_kernel<256, 256, 128, 5, false>", "gemm_i8_dma_kernel<256, 192, 128, 5, false>",
        "gemm_i8_dma_kernel<256, 128, 128, 6, false>", "gemm_i8_dma_kernel<128, 128, 128, 10, false>"},
       {"gemm_i8_dma_kernel<256, 256, 128, 5, true>", "gemm_i8_dma_kernel<256, 192, 128, 5, true>",
        "gemm_i8_dma_kernel<256, 128, 128, 6, true>", "gemm_i8_dma_kernel<128, 128, 128, 10, true>"}},
      {{"gemm_i8_dma_kernel<256, 256, 64, 10, false>", "gemm_i8_kernel<256, 192, false>",
        "gemm_i8_dma_kernel<256, 128, 64, 10, false>", "gemm_i8_dma_kernel<128, 128, 64, 10, false>"},
       {"gemm_i8_dma_kernel<256, 256, 64, 10, true>", "gemm_i8_kernel<256, 192, true>",
        "gemm_i8_dma_kernel<256, 128, 64, 10, true>", "gemm_i8_dma_kernel<128, 128, 64, 10, true>"}},
      {{"gemm_i8_kernel<256, 256, false>", "gemm_i8_kernel<256, 192, false>", "gemm_i8_kernel<256, 128, false>",
        "gemm_i8_kernel<128, 128, false>"},
       {"gemm_i8_kernel<256, 256, true>", "gemm_i8_kernel<256, 192, true>", "gemm_i8_kernel<256, 128, true>",
        "gemm_i8_kernel<128, 128, true>"}}};
  const int c = bm == 128 ? 3 : (bn == 256 ? 0 : (bn == 192 ? 1 : 2));
  return names[pick_k(K)][grouped][c];
}

}  // namespace

hipError_t launch_scaled_mm(const GemmArgs& a, hipStream_t stream) {
  const TileCfg t = pick_tile(a.M, a.N, a.K);
  if (t.bm == 256 && t.bn == 256) return launch_tiles<256, 256, false>(a, 0, stream);
  if (t.bm == 256 && t.bn == 192) return launch_tiles<256, 192, false>(a, 0, stream);
  if (t.bm == 256) return launch_tiles<256, 128, false>(a, 0, stream);
  return launch_tiles<128, 128, false>(a, 0, stream);
}

const char* scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K) {
  const TileCfg t = pick_tile(M, N, K);
  return kernel_name(t.bm, t.bn, false, K);
}

constexpr int kFp8BlockStages = 2;  // stages of the block-scaled FP8 ring

// Rows of the block-scaled FP8 tile: 256 (8 waves, one workgroup per CU;
// 4-7% faster per tile than two 128-row workgroups) unless that leaves a
// last round of tiles less than three quarters full on a short grid
// (2048 x 4096 x 6144: 384 tiles of 256 rows, 83.4 us, against 78.2 on 768
// of 128).
int fp8_block_rows(int64_t M, int64_t N) {
  const int64_t t = ((M + 255) / 256) * ((N + 127) / 128), r = t % 256;
  return (t >= 1024 || r == 0 || r > 192) ? 256 : 128;
}

// W8A8 FP8: per-tensor / per-channel weight scales run the ring kernel when K
// is a multiple of 128 (the int8 tile menu), the register-staged FP8 kernel
// otherwise; 128 x 128 block scales run the block-scaled ring kernel when K
// is a multiple of 128, else the register-staged kernel with the per-block
// scaling on 128 x 128 tiles.
hipError_t launch_scaled_mm_fp8(const GemmArgs& a, bool block, hipStream_t stream) {
  const dim3 block_dim(256);
  if (block || a.K % 128 != 0) {
    const int tm = (int)((a.M + 127) / 128), tn = (int)((a.N + 127) / 128);
    if (block && a.K % 128 == 0) {
      if (fp8_block_rows(a.M, a.N) == 256) {
        const int tm2 = (int)((a.M + 255) / 256);
        hipLaunchKernelGGL((gemm_fp8_block_dma_kernel<kFp8BlockStages, 256>), dim3((unsigned)(tm2 * tn)), dim3(512), 0,
                           stream, a, tm2, tn);
      } else {
        hipLaunchKernelGGL((gemm_fp8_block_dma_kernel<kFp8BlockStages, 128>), dim3((unsigned)(tm * tn)), block_dim, 0,
                           stream, a, tm, tn);
      }
    } else if (block)
      hipLaunchKernelGGL((gemm_fp8_kernel<128, 128, true>), dim3((unsigned)(tm * tn)), block_dim, 0, stream, a, tm,
                         tn);
    else
      hipLaunchKernelGGL((gemm_fp8_kernel<128, 128, false>), dim3((unsigned)(tm * tn)), block_dim, 0, stream, a, tm,
                         tn);
    return hipGetLastError();
  }
  const TileCfg t = pick_tile(a.M, a.N, a.K);
  const int tm = (int)((a.M + t.bm - 1) / t.bm), tn = (int)((a.N + t.bn - 1) / t.bn);
  const dim3 grid((unsigned)(tm * tn));
  if (t.bm == 256 && t.bn == 256)
    hipLaunchKernelGGL((gemm_fp8_dma_kernel<256, 256, ring_halves<256, 256, 128>()>), grid, block_dim, 0, stream, a, tm,
                       tn);
  else if (t.bm == 256 && t.bn == 192)
    hipLaunchKernelGGL((gemm_fp8_dma_kernel<256, 192, ring_halves<256, 192, 128>()>), grid, block_dim, 0, stream, a, tm,
                       tn);
  else if (t.bm == 256)
    hipLaunchKernelGGL((gemm_fp8_dma_kernel<256, 128, ring_halves<256, 128, 128>()>), grid, block_dim, 0, stream, a, tm,
                       tn);
  else
    hipLaunchKernelGGL((gemm_fp8_dma_kernel<128, 128, ring_halves<128, 128, 128>()>), grid, block_dim, 0, stream, a, tm,
                       tn);
  return hipGetLastError();
}

const char* scaled_mm_fp8_kernel_name(int64_t M, int64_t N, int64_t K, bool block) {
  static_assert(kFp8BlockStages == 2, "the names below");
  if (block && K % 128 == 0)
    return fp8_block_rows(M, N) == 256 ? "gemm_fp8_block_dma_kernel<2, 256>" : "gemm_fp8_block_dma_kernel<2, 128>";
  if (block) return "gemm_fp8_kernel<128, 128, true>";
  if (K % 128 != 0) return "gemm_fp8_kernel<128, 128, false>";
  const TileCfg t = pick_tile(M, N, K);
  if (t.bm == 256 && t.bn == 256) return "gemm_fp8_dma_kernel<256, 256, 5>";
  if (t.bm == 256 && t.bn == 192) return "gemm_fp8_dma_kernel<256, 192, 5>";
  if (t.bm == 256) return "gemm_fp8_dma_kernel<256, 128, 6>";
  return "gemm_fp8_dma_kernel<128, 128, 10>";
}

hipError_t launch_grouped_mm(const GemmArgs& a, hipStream_t stream) {
  // one partial m-tile per expert on top of the full tiles
  return launch_tiles<256, 256, true>(a, a.E, stream);
}

const char* grouped_mm_kernel_name(int64_t K) { return kernel_name(256, 256, true, K); }

}  // namespace w8a8
