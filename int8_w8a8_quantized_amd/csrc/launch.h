// Host-side launchers of the libw8a8 kernels. They assume the arguments were
// validated by the C ABI layer (api.cpp) and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int mode,
                               const float* s_in, const int32_t* zp_in, int8_t* xq, int64_t ldq,
                               float* s_x, int32_t* zp, hipStream_t stream);

hipError_t launch_colsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw, const int32_t* zp_in,
                         int32_t* out, hipStream_t stream);

struct RequantParts {
  int32_t P;
  int64_t row_start[17];  // prefix sums of the logical widths, row_start[P] == N
};

hipError_t launch_requant_max(int8_t* W, int64_t N, int64_t K, int64_t ldw,
                              const float* part_scales, const RequantParts& parts, float* s_max,
                              int32_t* err_flag, hipStream_t stream);

hipError_t launch_expand_scales(const float* part_scales, const RequantParts& parts, int64_t N,
                                float* s_w, int32_t* err_flag, hipStream_t stream);

hipError_t launch_fp8_block_to_int8(const uint8_t* W8, const float* S, int64_t E, int64_t N,
                                    int64_t K, int8_t* Wq, float* s, int32_t* err_flag,
                                    hipStream_t stream);

// Everything the GEMM kernels read besides the two operands' base pointers.
struct GemmArgs {
  const int8_t* A;  // activations xq
  int64_t lda;
  const int8_t* B;  // weights Wq [N,K] (or [E,N,K])
  int64_t ldb;
  int64_t M, N, K;
  const float* s_x;
  int32_t sx_per_token;
  const float* s_w;
  int32_t sw_per_channel;
  const int32_t* zp;      // [M] per-token zero points (AZP_PER_TOKEN)
  const int32_t* colsum;  // [N] colsum (PER_TOKEN) or azp_adj (STATIC)
  int32_t azp_mode;
  const uint16_t* bias;
  void* out;
  int32_t out_i32;
  int64_t ldo;
  // grouped (MoE) extras
  const int32_t* row_ids;
  const int32_t* expert_offsets;
  int64_t E;
  int64_t M_src;
};

hipError_t launch_scaled_mm(const GemmArgs& a, hipStream_t stream);  // MFMA tiles, any M
// M <= 128: weight streaming. Some shapes split K over workgroups when a
// workspace of decode_workspace_bytes(M, N, K) bytes is given (no state is
// kept in it between calls); without it they run unsplit. From M = 65 on only
// the split form streams; every other shape runs launch_scaled_mm.
hipError_t launch_decode_mm(const GemmArgs& a, void* workspace, size_t ws_bytes, hipStream_t stream);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Name of the kernel instance launch_decode_mm / launch_scaled_mm runs for a shape.
const char* decode_kernel_name(int64_t M, int64_t N, int64_t K, size_t ws_bytes);
const char* scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K);
constexpr int64_t kDecodeMaxM = 128;
// Per-token symmetric quantisation of x (bf16 [M,K], ldx) fused with the
// decode GEMM in one launch when fused_linear_fits(M, N, K): out = the bf16 GEMM
// of a (a.A and a.s_x are not read; no zero points), and xq / s_x receive the
// codes and scales exactly as launch_quantize_act writes them.
bool fused_linear_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_fused_linear(const GemmArgs& a, const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldq,
                               float* s_x, hipStream_t stream);
const char* fused_linear_kernel_name(int64_t M, int64_t N, int64_t K);
hipError_t launch_grouped_mm(const GemmArgs& a, hipStream_t stream);
const char* grouped_mm_kernel_name(int64_t K);

// W8A8 FP8 (quant.hip, gemm.hip). mode: 0 per token, 1 per tensor (*s_in),
// 2 per token in groups of 128 along K (scales group-major [G, M]).
// RMS normalisation (after the optional residual add, residual updated in
// place) fused with the per-token symmetric quantiser; y optional.
hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                float eps, uint16_t* residual, int64_t ldr, uint16_t* y, int64_t ldy, int8_t* xq,
                                int64_t ldq, float* s_x, hipStream_t stream);
hipError_t launch_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int mode,
                                   const float* s_in, uint8_t* xq, int64_t ldq, float* s_x, hipStream_t stream);
// a.A / a.B hold E4M3 codes; out_i32 means a binary32 output; no zero points.
hipError_t launch_scaled_mm_fp8(const GemmArgs& a, bool block, hipStream_t stream);
const char* scaled_mm_fp8_kernel_name(int64_t M, int64_t N, int64_t K, bool block);

// MoE expert block steps (moe.hip). Routing needs moe_route_chunks(tokens) * E
// 64-bit masks of scratch; E <= 512, k <= min(E, 64).
int64_t moe_route_chunks(int64_t tokens);
hipError_t launch_moe_route(const float* logits, int64_t ldl, int64_t tokens, int E, int k, int32_t* ids,
                            float* wts, int32_t* row_ids, int32_t* offsets, int32_t* pos, uint64_t* masks,
                            hipStream_t stream);
// I % 8 == 0, I <= 16384; act (bf16 [T, I], ld_act) nullable.
hipError_t launch_silu_mul_quant(const uint16_t* h, int64_t T, int64_t I, int64_t ldh, int8_t* aq, int64_t ldq,
                                 float* s_a, uint16_t* act, int64_t ld_act, hipStream_t stream);
// N % 8 == 0, k <= 16.
hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* pos, const float* wts,
                              int64_t tokens, int k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t stream);

}  // namespace w8a8
