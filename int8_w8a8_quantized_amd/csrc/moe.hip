// The steps of the int8 MoE expert block around the grouped GEMM: routing,
// the expert sort, the activated product with its per-token requantisation,
// and the weighted combine. The block is the int8 MoE method of
// "MiniMax-M2.7 FP8 转昆仑芯 INT8" (版本: experts w1 / w2 / w3, w1 and w3 fused
// into one w13, per-token dynamic symmetric int8 activations, per-channel
// symmetric int8 weights) and the w8a8 int8 MoE scheme of "[SGLang] W4A8,
// W8A8, W4A4: 혼합 정밀도 양자화 스킴" (구조도).
//
// Routing (moe_topk_kernel): one wave per token, lane l holding the logits of
// experts l, l + 64, ... Each expert is ranked by counting the experts that
// beat it (a larger logit, or an equal one and a lower index); the k ranked
// first are the selection, in rank order. The weights are the softmax of the k selected
// logits. Tokens are taken 64 at a time per workgroup (a chunk); for each
// expert the workgroup publishes a 64-bit mask of the chunk's tokens routed
// to it.
// Sort (moe_scatter_kernel): pairs are ordered by expert, then token. The
// sorted row of the pair (token t of chunk c, expert e) is the start of e's
// rows + the tokens routed to e in the chunks before c + the tokens of chunk
// c before t that are routed to e -- all popcounts of the masks, so the order
// is fixed without atomics.
// Activated product (silu_mul_quant_kernel): silu(gate) * up in binary32 from
// the bf16 w13 output, rounded to bf16 (the dtype the product has between
// the two GEMMs), then the per-token symmetric quantiser's rule and exact
// rounding on those bf16 values.
// Combine (moe_combine_kernel): out[t] = sum_j w[t, j] * y[pos[t, j]], fused
// multiply-adds in binary32 in the order j = 0, 1, ..., rounded to bf16
// (k <= 16).

#include "launch.h"
#include "quant_common.h"

namespace w8a8 {

constexpr int kRouteChunk = 32;  // tokens per routing workgroup (at most 64: one 64-bit mask per expert)

// Order-preserving map of a float onto unsigned integers (larger float ->
// larger integer; -0 and +0 apart, which does not matter for a maximum).
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


constexpr int kRouteWaves = 16;  // waves per routing workgroup: 2 tokens each

// Each wave ranks its tokens' experts: 64-bit keys (the logit mapped to an
// order-preserving integer above the complement of the expert index, so a
// larger key is a larger logit or an equal one with a lower index) go to
// the wave's LDS row, and every lane counts, for each of its experts, the
// larger keys, reading the row as broadcast 16-byte loads. The experts
// ranked below k are the selection, in rank order; no chain of cross-lane
// reductions is involved.
template <int EPL>
__global__ __launch_bounds__(64 * kRouteWaves) void moe_topk_kernel(const float* __restrict__ logits, int64_t ldl,
                                                                     int64_t tokens, int E, int k,
                                                                     int32_t* __restrict__ ids,
                                                                     float* __restrict__ wts,
                                                                     uint64_t* __restrict__ masks) {
  constexpr int EP = 64 * EPL;
  __shared__ unsigned long long mask[EP];
  __shared__ __attribute__((aligned(16))) uint64_t kbuf[kRouteWaves][EP];
  __shared__ float topv[kRouteWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 64 * kRouteWaves) mask[e] = 0ull;
  __syncthreads();
  // the wave's tokens lt = wave, wave + 16, ...: every logit load is issued
  // before the first token is ranked
  constexpr int TPW = kRouteChunk / kRouteWaves;
  float lv[TPW][EPL];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = c * kRouteChunk + wave + kRouteWaves * i;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      lv[i][q] = (t < tokens && e < E) ? logits[t * ldl + e] : 0.0f;
    }
  }
  uint64_t* kw = kbuf[wave];
  const int E2 = (E + 1) & ~1;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int lt = wave + kRouteWaves * i;
    const int64_t t = c * kRouteChunk + lt;
    if (t >= tokens) break;
    uint64_t key[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      key[q] = ((uint64_t)float_key(lv[i][q]) << 32) | (uint32_t)~(uint32_t)e;
      if (e < E2) kw[e] = e < E ? key[q] : 0ull;  // the padding key loses to every expert
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own LDS writes, in order
    int rank[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) rank[q] = 0;
    for (int e0 = 0; e0 < E2; e0 += 2) {
      const ulonglong2 o = *reinterpret_cast<const ulonglong2*>(kw + e0);
#pragma unroll
      for (int q = 0; q < EPL; ++q) rank[q] += (o.x > key[q] ? 1 : 0) + (o.y > key[q] ? 1 : 0);
    }
    // the winner's logit, then the softmax over the k selected
#pragma unroll
    for (int q = 0; q < EPL; ++q)
      if (lane + 64 * q < E && rank[q] == 0) topv[wave] = lv[i][q];
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float top = topv[wave];
    float ex[EPL], part = 0.0f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const bool sel = lane + 64 * q < E && rank[q] < k;
      ex[q] = sel ? expf(lv[i][q] - top) : 0.0f;
      part += ex[q];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, kWave);
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      if (e < E && rank[q] < k) {
        ids[t * k + rank[q]] = e;
        wts[t * k + rank[q]] = ex[q] / part;
        atomicOr(&mask[e], 1ull << lt);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64 * kRouteWaves) masks[c * E + e] = mask[e];
}

template <int EPL>
__global__ __launch_bounds__(1024) void moe_scatter_kernel(const int32_t* __restrict__ ids,
                                                           const uint64_t* __restrict__ masks, int64_t tokens,
                                                           int E, int k, int64_t nchunks,
                                                           int32_t* __restrict__ row_ids,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pos) {
  constexpr int NT = 1024, U = 4;
  __shared__ int total[64 * EPL], before[64 * EPL], start[64 * EPL + 1];
  __shared__ unsigned long long own[64 * EPL];
  const int64_t c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += NT) {
    total[e] = 0;
    before[e] = 0;
    own[e] = masks[c * E + e];
  }
  __syncthreads();
  // routed tokens per expert over all chunks, and over the chunks before this
  // one: U mask loads in flight per thread, then their popcounts
  const int64_t cells = nchunks * E;
  for (int64_t i0 = threadIdx.x; i0 < cells; i0 += (int64_t)NT * U) {
    uint64_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT;
      m[u] = i < cells ? masks[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT;
      const int n = __popcll(m[u]);
      if (n) {
        const int e = (int)(i % E);
        atomicAdd(&total[e], n);
        if (i / E < c) atomicAdd(&before[e], n);
      }
    }
  }
  __syncthreads();
  // exclusive prefix of the totals over the experts (wave 0, 64 at a time)
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const int v = e < E ? total[e] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      if (e < E) start[e] = carry + incl - v;
      carry += __shfl(incl, 63, kWave);
    }
    if (lane == 0) start[E] = carry;
  }
  __syncthreads();
  if (c == 0)
    for (int e = threadIdx.x; e <= E; e += NT) offsets[e] = start[e];
  // every routed pair of this chunk
  for (int p = threadIdx.x; p < kRouteChunk * k; p += NT) {
    const int lt = p / k;
    const int64_t t = c * kRouteChunk + lt;
    if (t >= tokens) break;
    const int e = ids[t * k + (p % k)];
    const int rank = __popcll(own[e] & ((1ull << lt) - 1ull));
    const int r = start[e] + before[e] + rank;
    row_ids[r] = (int32_t)t;
    pos[t * k + (p % k)] = r;
  }
}

// silu(g) = g / (1 + exp(-g)) in binary32, written as g e' / (1 + e) with
// e = exp(-|g|) and e' = 1 (g >= 0) or e (g < 0), so no exponential overflows.
// e = 2^(a log2 e) for a = -|g|: the product is split into its rounded value
// t (log2 e in two parts) and the exact remainder r, e = 2^t (1 + r ln 2) from
// the hardware exp2 (v_exp_f32), and the quotient uses the hardware reciprocal
// (v_rcp_f32): a few units in the last place of binary32 in all, against the
// 2^16 units between neighbouring bf16 values the result is rounded to.
__device__ __forceinline__ float silu(float g) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;  // binary32 log2(e)
  constexpr float kLog2eLo = 1.92596298909109e-8f;        // log2(e) - kLog2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float a = -fabsf(g);
  const float t = a * kLog2eHi;
  const float r = fmaf(a, kLog2eHi, -t) + a * kLog2eLo;
  const float p = __builtin_amdgcn_exp2f(t);
  const float e = fmaf(p, r * kLn2, p);
  return (g >= 0.0f ? g : g * e) * __builtin_amdgcn_rcpf(1.0f + e);
}

// silu(g) * u, rounded to bf16 (both halves of the result word).
__device__ __forceinline__ uint32_t silu_mul_pair(uint32_t g2, uint32_t u2) {
  return pack_bf16x2(silu(bf16_lo(g2)) * bf16_lo(u2), silu(bf16_hi(g2)) * bf16_hi(u2));
}

// TPR threads own one row of the w13 output (several rows per 256-thread
// workgroup when TPR = 64); CH 8-element chunks of the activated product per
// thread, kept in registers between the absmax and the encoding.
template <int TPR, int CH>
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(const uint16_t* __restrict__ h, int64_t T,
                                                             int64_t I, int64_t ldh, int8_t* __restrict__ aq,
                                                             int64_t ldq, float* __restrict__ s_a,
                                                             uint16_t* __restrict__ act, int64_t ld_act) {
  constexpr int RPB = 256 / TPR, WPR = TPR / 64;
  const int sub = threadIdx.x % TPR;
  const int64_t t = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool row_ok = t < T;
  if (WPR == 1 && !row_ok) return;
  const int64_t nchunk = I >> 3;
  const uint16_t* gate = h + (row_ok ? t : 0) * ldh;
  const uint16_t* up = gate + I;
  uint4 g[CH], u[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    const bool ok = row_ok && j < nchunk;
    g[c] = ok ? ld16(gate + j * 8) : make_uint4(0, 0, 0, 0);
    u[c] = ok ? ld16(up + j * 8) : make_uint4(0, 0, 0, 0);
  }
  uint4 a[CH];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    a[c] = make_uint4(silu_mul_pair(g[c].x, u[c].x), silu_mul_pair(g[c].y, u[c].y),
                      silu_mul_pair(g[c].z, u[c].z), silu_mul_pair(g[c].w, u[c].w));
    absmax8(a[c], amax);
  }
  amax = wave_extreme<true>(amax);
  if (WPR > 1) {
    __shared__ float red[RPB][WPR > 1 ? WPR : 1];
    const int rb = threadIdx.x / TPR;
    if ((threadIdx.x & 63) == 0) red[rb][sub >> 6] = amax;
    __syncthreads();
    amax = red[rb][0];
#pragma unroll
    for (int i = 1; i < WPR; ++i) amax = max_ieee(amax, red[rb][i]);
  }
  if (!row_ok) return;
  const RowParams p = row_params<kDynSym>(-amax, amax, nullptr, nullptr);
  if (sub == 0) s_a[t] = p.s;
  int8_t* orow = aq + t * ldq;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t j = (int64_t)c * TPR + sub;
    if (j < nchunk) {
      *reinterpret_cast<uint2*>(orow + j * 8) = codes8<kDynSym>(a[c], p);
      if (act) st16(act + t * ld_act + j * 8, a[c]);
    }
  }
}

// One wave per token; lane l takes the 8-element chunks l, l + 64, ... of the
// row, with the k expert rows of a chunk loaded together. KMAX >= k bounds
// the registers held for them.
template <int KMAX>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ y, int64_t ldy,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ wts, int64_t tokens, int k,
                                                          int64_t N, uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const uint16_t* src[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool live = j < k;
    src[j] = y + (live ? (int64_t)pos[t * k + j] : 0) * ldy;
    w[j] = live ? wts[t * k + j] : 0.0f;
  }
  const int64_t nchunk = N >> 3;
  uint16_t* orow = out + t * ldo;
  for (int64_t c = lane; c < nchunk; c += 64) {
    uint4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) v[j] = ld16(src[j] + c * 8);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(w[j], bf16_lo(q[i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(w[j], bf16_hi(q[i]), acc[2 * i + 1]);
        }
      }
    }
    st16(orow + c * 8, make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])));
  }
}

int64_t moe_route_chunks(int64_t tokens) { return (tokens + kRouteChunk - 1) / kRouteChunk; }

hipError_t launch_moe_route(const float* logits, int64_t ldl, int64_t tokens, int E, int k, int32_t* ids,
                            float* wts, int32_t* row_ids, int32_t* offsets, int32_t* pos, uint64_t* masks,
                            hipStream_t stream) {
  const int64_t nch = moe_route_chunks(tokens);
  const dim3 grid((unsigned)nch), block(64 * kRouteWaves), block_s(1024);
#define W8A8_ROUTE(EPLV)                                                                                      \
  do {                                                                                                      \
    hipLaunchKernelGGL((moe_topk_kernel<EPLV>), grid, block, 0, stream, logits, ldl, tokens, E, k, ids, wts,  \
                       masks);                                                                              \
    hipError_t e = hipGetLastError();                                                                       \
    if (e != hipSuccess) return e;                                                                          \
    hipLaunchKernelGGL((moe_scatter_kernel<EPLV>), grid, block_s, 0, stream, ids, masks, tokens, E, k, nch, \
                       row_ids, offsets, pos);                                                              \
    return hipGetLastError();                                                                               \
  } while (0)
  if (E <= 64) W8A8_ROUTE(1);
  if (E <= 128) W8A8_ROUTE(2);
  if (E <= 256) W8A8_ROUTE(4);
  W8A8_ROUTE(8);
#undef W8A8_ROUTE
}

hipError_t launch_silu_mul_quant(const uint16_t* h, int64_t T, int64_t I, int64_t ldh, int8_t* aq, int64_t ldq,
                                 float* s_a, uint16_t* act, int64_t ld_act, hipStream_t stream) {
  const int64_t nchunk = I / 8;
  const int tpr = nchunk <= 64 * 4 ? 64 : 256;
  const int ch = (int)((nchunk + tpr - 1) / tpr);  // <= 8 for I <= 16384
  const dim3 block(256);
#define W8A8_SMQ(TPRV, CHV)                                                                                 \
  hipLaunchKernelGGL((silu_mul_quant_kernel<TPRV, CHV>), dim3((unsigned)((T + 256 / TPRV - 1) / (256 / TPRV))), \
                     block, 0, stream, h, T, I, ldh, aq, ldq, s_a, act, ld_act)
  if (tpr == 64) {
    if (ch <= 1) W8A8_SMQ(64, 1);
    else if (ch <= 2) W8A8_SMQ(64, 2);
    else if (ch <= 3) W8A8_SMQ(64, 3);
    else W8A8_SMQ(64, 4);
  } else {
    if (ch <= 2) W8A8_SMQ(256, 2);
    else if (ch <= 4) W8A8_SMQ(256, 4);
    else W8A8_SMQ(256, 8);
  }
#undef W8A8_SMQ
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* pos, const float* wts,
                              int64_t tokens, int k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t stream) {
  const dim3 grid((unsigned)((tokens + 3) / 4)), block(256);
#define W8A8_COMB(KV) \
  hipLaunchKernelGGL((moe_combine_kernel<KV>), grid, block, 0, stream, y, ldy, pos, wts, tokens, k, N, out, ldo)
  if (k <= 1) W8A8_COMB(1);
  else if (k <= 2) W8A8_COMB(2);
  else if (k <= 4) W8A8_COMB(4);
  else if (k <= 8) W8A8_COMB(8);
  else W8A8_COMB(16);
#undef W8A8_COMB
  return hipGetLastError();
}

}  // namespace w8a8
