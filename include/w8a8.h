/*
 * w8a8.h -- C ABI of libw8a8.so, the W8A8 INT8 linear layer for AMD MI355X (gfx950).
 *
 * The layer, as the three source pages describe it:
 *   [vLLM]   "vLLM INT8 W8A8 量化实战：用 llm-compressor 制作 8 位权重与 8 位激活的推理模型"
 *   [SGLang] "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴"
 *   [Kunlun] "MiniMax-M2.7 FP8 转昆仑芯 INT8"
 * quantises bf16 activations to int8 (per token and dynamic, symmetric or with
 * a zero point, or with a static per-tensor scale), multiplies them with int8
 * weights into exact int32 sums, and applies token scale, weight scale,
 * zero-point correction and bias in a fused epilogue that writes bf16
 * ([SGLang] 핵심 코드 분석 §3-§4). Load-time preparation (column sums,
 * requantise to the max per-tensor scale, FP8 block -> per-row int8) and an
 * MoE grouped GEMM complete it.
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless marked "host". Every buffer is owned
 *    by the caller; the library allocates no device memory at run time and
 *    keeps no state besides a per-device property cache and, for
 *    w8a8_scaled_mm_int8_noalloc, one static scratch array per GPU.
 *  - "stream" is a hipStream_t (NULL = the null stream). Work is enqueued
 *    asynchronously on it; nothing synchronises.
 *  - Matrices are row-major; ld* are row strides in elements.
 *  - bf16 values travel as their uint16_t bit patterns.
 *  - Shape, null-pointer, alignment and range problems are found on the host
 *    and returned before anything is enqueued (W8A8_ERR_INVALID_ARG); a
 *    combination the layer does not define returns W8A8_ERR_NOT_IMPLEMENTED
 *    (the [vLLM] 4.3 behaviour for an unmatched scheme); a failed launch
 *    returns W8A8_ERR_HIP. Data-dependent problems (an illegal scale, an FP8
 *    NaN code) are OR-ed into a caller's device err_flag word, to be read
 *    after synchronising; the other outputs are then unspecified.
 *  - Empty problems (a zero M, N, E or T) are legal no-ops.
 *  - The calls are reentrant; w8a8_last_error() is per host thread.
 *  - NaN or infinite activations are outside the contract.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w8a8_status {
  W8A8_OK = 0,
  W8A8_ERR_INVALID_ARG = 1,
  W8A8_ERR_NOT_IMPLEMENTED = 2,
  W8A8_ERR_UNSUPPORTED_DEVICE = 3,
  W8A8_ERR_HIP = 4
} w8a8_status;

/* Quantisation strategies ([SGLang] 설계 근거: TENSOR/CHANNEL/BLOCK/TOKEN/GROUP). */
enum {
  W8A8_STRATEGY_TENSOR = 0,
  W8A8_STRATEGY_CHANNEL = 1,
  W8A8_STRATEGY_TOKEN = 2,
  W8A8_STRATEGY_BLOCK = 3,
  W8A8_STRATEGY_GROUP = 4
};

/* Activation quantisation modes of w8a8_quantize_act. */
enum {
  W8A8_QUANT_DYN_SYM = 0,     /* per token, s = absmax/127, codes [-127,127]        */
  W8A8_QUANT_DYN_ASYM = 1,    /* per token, zero point, codes [-128,127]            */
  W8A8_QUANT_STATIC_SYM = 2,  /* one calibrated s_in, codes [-127,127]              */
  W8A8_QUANT_STATIC_ASYM = 3  /* one calibrated s_in and zp_in, codes [-128,127]    */
};

/* Zero-point correction applied by the GEMM epilogue. */
enum {
  W8A8_AZP_NONE = 0,
  W8A8_AZP_PER_TOKEN = 1,  /* c = acc - zp[t] * colsum[n]   (dynamic asymmetric) */
  W8A8_AZP_STATIC = 2      /* c = acc - azp_adj[n]          (static asymmetric)  */
};

/* Output element type of the GEMMs. */
enum {
  W8A8_OUT_BF16 = 0, /* bf16(c * s_x * s_w + bias), round to nearest even            */
  W8A8_OUT_I32 = 1,  /* the corrected integer c itself (exact; for checking)        */
  W8A8_OUT_F32 = 2   /* w8a8_scaled_mm_fp8 only: the binary32 value before rounding */
};

/* W8A8 FP8 activation quantisation (w8a8_quantize_act_fp8). */
enum {
  W8A8_FP8_ACT_TOKEN = 0,    /* per token, s = absmax / 448                        */
  W8A8_FP8_ACT_TENSOR = 1,   /* one given scale                                    */
  W8A8_FP8_ACT_GROUP128 = 2  /* per token in groups of 128 along K                 */
};

/* W8A8 FP8 weight scales (w8a8_scaled_mm_fp8). */
enum {
  W8A8_FP8_W_TENSOR = 0,   /* one scale                                              */
  W8A8_FP8_W_CHANNEL = 1,  /* one per output channel [N]                             */
  W8A8_FP8_W_BLOCK128 = 2  /* one per 128 x 128 block [ceil(N/128), ceil(K/128)]     */
};

/* err_flag bits. */
enum {
  W8A8_FLAG_NAN_CODE = 1,  /* an FP8 NaN code (0x7F or 0xFF) in a weight              */
  W8A8_FLAG_BAD_SCALE = 2, /* a scale that is NaN, infinite or negative (or not > 0
                              where the call says so)                              */
  W8A8_FLAG_NONFINITE = 4  /* a dequantised weight overflowed float32               */
};

/* Largest K any call accepts: |acc - zp*colsum| <= 2*K*128*127 stays below 2^31. */
#define W8A8_MAX_K 65536
/* Largest number of partitions of a fused weight in w8a8_prepare_requant_max. */
#define W8A8_MAX_PARTITIONS 16
/* Bytes of the static scratch array behind w8a8_scaled_mm_int8_noalloc (8 MiB,
 * one per GPU): the largest w8a8_scaled_mm_workspace_size of any shape. */
#define W8A8_NOALLOC_SCRATCH_BYTES (8 << 20)

/* The quantisation scheme of one linear layer, as its checkpoint declares it
 * ([vLLM] 4.1: bit widths, strategy, dynamic flag and symmetry of the weight
 * and of the input). */
typedef struct w8a8_scheme {
  int32_t weight_bits;      /* must be 8                                   */
  int32_t input_bits;       /* must be 8                                   */
  int32_t weight_strategy;  /* W8A8_STRATEGY_TENSOR or _CHANNEL            */
  int32_t input_strategy;   /* _TENSOR (static) or _TOKEN (dynamic)        */
  int32_t weight_symmetric; /* must be 1                                   */
  int32_t input_symmetric;  /* 0 or 1                                      */
  int32_t weight_dynamic;   /* must be 0                                   */
  int32_t input_dynamic;    /* 0 with _TENSOR input, 1 with _TOKEN input   */
} w8a8_scheme;

/* Check that `device` is a gfx950 GPU and cache its properties. Every other
 * call performs the same check lazily on the current device; this one lets a
 * caller fail early. (The analogue of the minimum-capability gate of
 * [vLLM] 一.) Returns W8A8_ERR_UNSUPPORTED_DEVICE for any other GPU. */
w8a8_status w8a8_init(int device);

/* Validate a scheme against the combinations the layer defines ([vLLM] 4.1
 * table: both 8-bit; weight per-tensor or per-channel, static and symmetric;
 * input either static per-tensor or dynamic per-token, symmetric or not).
 * On success writes the activation mode (W8A8_QUANT_*) to *quant_mode and the
 * kernel variant flags to *is_channelwise (both nullable). Anything else
 * returns W8A8_ERR_NOT_IMPLEMENTED and w8a8_last_error() names the fields. */
w8a8_status w8a8_check_scheme(const w8a8_scheme* scheme, int32_t* quant_mode,
                              int32_t* is_channelwise);

/* Quantise bf16 activations x [M,K] (row stride ldx) to int8 xq [M,K]
 * (row stride ldq). [SGLang] 핵심 코드 분석 §3 (per-token quantiser) with the
 * per-row rule of [Kunlun] 转换关系; [vLLM] 4.1-4.2 for the static modes.
 *   DYN_SYM:     s_x[t] = max|x_t|/127, xq = clamp(rne(x/s_x[t]), -127, 127);
 *                an all-zero row gives s_x = 1, xq = 0.
 *   DYN_ASYM:    lo = min(0, min x_t), hi = max(0, max x_t),
 *                s_x[t] = (hi-lo)/255, zp[t] = clamp(-128 - rne(lo/s), -128, 127),
 *                xq = clamp(rne(x/s) + zp[t], -128, 127); all-zero row: 1, 0, 0.
 *   STATIC_SYM:  xq = clamp(rne(x / *s_in), -127, 127).
 *   STATIC_ASYM: xq = clamp(rne(x / *s_in) + *zp_in, -128, 127).
 * Every float step is one IEEE binary32 operation (true division, round to
 * nearest even), so the codes are exactly determined.
 * s_x: float [M], written in the dynamic modes (else ignored, may be NULL).
 * zp: int32 [M], written in DYN_ASYM (else may be NULL).
 * s_in / zp_in: device scalars read in the static modes (else may be NULL);
 * zp_in is an int8 zero point, in [-128, 127] (outside that range the codes
 * are unspecified).
 * Requires K % 16 == 0, K <= W8A8_MAX_K, x and xq 16-byte aligned,
 * ldx % 8 == 0, ldq % 16 == 0, ldx >= K, ldq >= K. */
w8a8_status w8a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              int32_t mode, const float* s_in, const int32_t* zp_in,
                              int8_t* xq, int64_t ldq, float* s_x, int32_t* zp,
                              void* stream);

/* Column sums of an int8 weight W [N,K] (row stride ldw):
 * out[n] = sum_k W[n,k], or zp_in * sum_k W[n,k] when zp_in (a device int32
 * scalar) is given -- the azp_adj of [SGLang] 핵심 코드 분석 §4 for the static
 * asymmetric scheme. Run it after any requantisation of W.
 * Requires K % 16 == 0, K <= W8A8_MAX_K, W 16-byte aligned, ldw % 16 == 0. */
w8a8_status w8a8_prepare_colsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw,
                                const int32_t* zp_in, int32_t* out, void* stream);

/* Requantise, in place, a fused weight W [N,K] whose P row partitions
 * (host array logical_widths [P], summing to N) each carry one per-tensor
 * scale (device part_scales [P]) to the single largest scale
 * ([SGLang] 핵심 코드 분석 §7, requantize_with_max_scale):
 *   s_max = max_p part_scales[p];  for the rows of partition p:
 *   W' = clamp(rne(fp32(W * s_p) / s_max), -128, 127).
 * Writes s_max to the device scalar *s_max. A scale that is not finite and
 * > 0 sets W8A8_FLAG_BAD_SCALE in *err_flag (device int32, nullable; the
 * call only ORs bits into it). 1 <= P <= W8A8_MAX_PARTITIONS; W 16-byte
 * aligned, ldw % 16 == 0, K % 16 == 0. */
w8a8_status w8a8_prepare_requant_max(int8_t* W, int64_t N, int64_t K, int64_t ldw,
                                     const float* part_scales,
                                     const int64_t* logical_widths /* host */, int32_t P,
                                     float* s_max, int32_t* err_flag, void* stream);

/* Expand the per-tensor scales of a fused weight's P row partitions (device
 * part_scales [P], host logical_widths [P] summing to N) into per-output-
 * channel scales s_w [N] (device): s_w[n] = part_scales[p] for the rows n of
 * partition p. With s_w_per_channel = 1 the GEMM then applies each
 * partition's own scale, so the fused weight needs no requantisation: the
 * lossless alternative to w8a8_prepare_requant_max for the fused partitions
 * that [SGLang] 핵심 코드 분석 §7 tracks through logical_widths (the page's
 * is_channelwise flag, §4, selects the per-channel path). A scale that is
 * not finite and > 0 sets W8A8_FLAG_BAD_SCALE in *err_flag (device int32,
 * nullable). 1 <= P <= W8A8_MAX_PARTITIONS; zero-width partitions are legal. */
w8a8_status w8a8_prepare_expand_scales(const float* part_scales,
                                       const int64_t* logical_widths /* host */, int32_t P,
                                       int64_t N, float* s_w, int32_t* err_flag, void* stream);

/* Convert E FP8 E4M3FN weights W8 [E,N,K] (OCP encoding) with float block
 * scales S [E, ceil(N/128), ceil(K/128)] to per-row symmetric int8
 * ([Kunlun] 转换关系):
 *   W32 = fp32(dec(W8[i,j]) * S[i/128, j/128])   (the scale multiplies)
 *   s[e,i] = fp32(max_j |W32[i,j]| / 127);  Wq = clamp(rne(W32 / s), -127, 127)
 * and an all-zero row gives Wq = 0, s = 1. Wq int8 [E,N,K], s float [E,N].
 * err_flag (device int32, required) receives W8A8_FLAG_NAN_CODE,
 * W8A8_FLAG_BAD_SCALE (NaN, infinite or negative block scale; zero is legal)
 * and W8A8_FLAG_NONFINITE bits. Requires K % 16 == 0, K <= W8A8_MAX_K and
 * 16-byte aligned W8 and Wq; rows are dense (row stride K). */
w8a8_status w8a8_prepare_fp8_block_to_int8(const uint8_t* W8, const float* S, int64_t E,
                                           int64_t N, int64_t K, int8_t* Wq, float* s,
                                           int32_t* err_flag, void* stream);

/* Bytes of workspace w8a8_scaled_mm_int8 can use for this shape (0 when it
 * uses none). With at least this many bytes, decode shapes (M <= 128) with a
 * long K split K over workgroups and add the ranges in a second kernel; with
 * fewer (or NULL) the call runs unsplit, with the same result. No state is
 * kept in it between calls, so any buffer serves; calls that may run at the
 * same time (other streams) need buffers of their own. */
size_t w8a8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K);

/* The scaled int8 GEMM with its fused epilogue ([SGLang] 핵심 코드 분석 §3-§4):
 *   acc[t,n] = sum_k xq[t,k] * Wq[n,k]        (exact int32)
 *   c = acc - zp[t]*colsum[n]   (azp_mode W8A8_AZP_PER_TOKEN)
 *     = acc - azp_adj[n]        (W8A8_AZP_STATIC)
 *     = acc                     (W8A8_AZP_NONE)
 *   out[t,n] = bf16(c * s_x[t or 0] * s_w[n or 0] + bias[n])   (W8A8_OUT_BF16)
 *            = c                                               (W8A8_OUT_I32)
 * xq int8 [M,K] (ldx), Wq int8 [N,K] (ldw; the [vLLM] 4.2 layout
 * [out_features, in_features]); s_x float [M] if s_x_per_token else [1];
 * s_w float [N] if s_w_per_channel else [1]; zp int32 [M] and colsum int32 [N]
 * (PER_TOKEN), or azp_adj int32 [N] (STATIC) -- pass it as `colsum`;
 * bias bf16 [N] or NULL; out bf16 or int32 [M,N] (ldo).
 * PER_TOKEN expects int8 zero points (zp in [-128, 127], as w8a8_quantize_act
 * writes them) and column sums of the int8 weight (|colsum| <= 2^23, which
 * every K <= W8A8_MAX_K gives); the result is unspecified outside that range.
 * workspace: device memory, 16-byte aligned, see w8a8_scaled_mm_workspace_size.
 * Requires K % 16 == 0, 1 <= K <= W8A8_MAX_K, xq/Wq/out 16-byte aligned,
 * ldx % 16 == 0, ldw % 16 == 0, ld* >= the row length. */
w8a8_status w8a8_scaled_mm_int8(const int8_t* xq, int64_t M, int64_t K, int64_t ldx,
                                const int8_t* Wq, int64_t N, int64_t ldw,
                                const float* s_x, int32_t s_x_per_token,
                                const float* s_w, int32_t s_w_per_channel,
                                const int32_t* zp, const int32_t* colsum, int32_t azp_mode,
                                const uint16_t* bias, void* out, int32_t out_dtype,
                                int64_t ldo, void* workspace, size_t workspace_bytes,
                                void* stream);

/* w8a8_scaled_mm_int8 without a workspace argument and without allocating,
 * for callers that cannot allocate device memory around the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, requirements and results as w8a8_scaled_mm_int8 given a
 * workspace of w8a8_scaled_mm_workspace_size(M, N, K) bytes: the split-K
 * partial tiles of the decode shapes go to a static device array of
 * W8A8_NOALLOC_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends (its address is looked up in w8a8_init, or on the first call
 * on a device). A shape that would need more scratch than that returns
 * W8A8_ERR_INVALID_ARG (no valid shape does today). Every call on one GPU
 * shares that GPU's array and it keeps the last call's contents: calls that
 * may overlap on one GPU (several streams, several host threads) race and
 * must be ordered by the caller. Nothing in the array needs to start at zero. */
w8a8_status w8a8_scaled_mm_int8_noalloc(const int8_t* xq, int64_t M, int64_t K, int64_t ldx,
                                        const int8_t* Wq, int64_t N, int64_t ldw,
                                        const float* s_x, int32_t s_x_per_token,
                                        const float* s_w, int32_t s_w_per_channel,
                                        const int32_t* zp, const int32_t* colsum,
                                        int32_t azp_mode, const uint16_t* bias, void* out,
                                        int32_t out_dtype, int64_t ldo, void* stream);

/* The dynamic per-token symmetric linear layer in one call: w8a8_quantize_act
 * (W8A8_QUANT_DYN_SYM) of x into xq / s_x, then w8a8_scaled_mm_int8 with
 * s_x per token, no zero points and a bf16 out -- the per-token quantiser
 * followed by the scaled GEMM of [SGLang] 핵심 코드 분석 §3, with the
 * quantiser fused into the GEMM's prologue as the same page's data flow
 * (quantise right before the GEMM) allows. Results are identical to the two
 * calls: xq int8 [M,K] (ldq) and s_x float [M] are written as
 * w8a8_quantize_act writes them (both caller-owned and required), out bf16
 * [M,N] (ldo) as w8a8_scaled_mm_int8 writes it. For M <= 2, N <= 4096,
 * K % 128 == 0 and M * K <= 16384 it is one kernel, in which every
 * workgroup quantises the activation itself (where that measured faster
 * than two launches); otherwise the two launches run in order on the
 * stream. x bf16 [M,K] (ldx % 8 == 0), Wq int8 [N,K] (ldw % 16 == 0),
 * s_w float [N] if s_w_per_channel else [1], bias bf16 [N] or NULL;
 * workspace as for w8a8_scaled_mm_int8. Requires K % 16 == 0,
 * 1 <= K <= W8A8_MAX_K, x/xq/Wq/out 16-byte aligned, ldq % 16 == 0. With
 * N == 0 only xq and s_x are written. */
w8a8_status w8a8_linear_dyn_sym(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const int8_t* Wq, int64_t N, int64_t ldw, const float* s_w,
                                int32_t s_w_per_channel, const uint16_t* bias, uint16_t* out,
                                int64_t ldo, int8_t* xq, int64_t ldq, float* s_x, void* workspace,
                                size_t workspace_bytes, void* stream);

/* The per-token quantiser fused into the op before it in a decoder layer
 * (the quantiser runs right before the GEMM: "[SGLang] W4A8, W8A8, W4A4:
 * 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3): RMS normalisation of bf16 rows,
 * after an optional residual add, then W8A8_QUANT_DYN_SYM on its bf16 output:
 *   h = residual ? bf16(x + residual) : x     (residual <- h, in place)
 *   y = bf16(h * gamma / sqrt(mean_k(h^2) + eps))
 *   s_x[t] = max|y_t| / 127,  xq = clamp(rne(y / s_x[t]), -127, 127)
 * (each bf16 value the correctly rounded one; the mean square, root and
 * products in binary64; the codes and the scale with the rule and exact
 * rounding of w8a8_quantize_act). x, residual (nullable) and y (nullable:
 * receives the normalised rows) bf16 [M, K] with strides ldx, ldr, ldy
 * (multiples of 8); gamma bf16 [K]; xq int8 [M, K] (ldq % 16 == 0), s_x
 * float [M]. K % 16 == 0; eps finite and > 0; x, residual, y, gamma and xq
 * 16-byte aligned. residual and y may be x itself, but not each other
 * (W8A8_ERR_INVALID_ARG). */
w8a8_status w8a8_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const uint16_t* gamma, float eps, uint16_t* residual, int64_t ldr,
                               uint16_t* y, int64_t ldy, int8_t* xq, int64_t ldq, float* s_x,
                               void* stream);

/* Grouped (MoE) scaled GEMM: the rows of the expert-sorted activation are
 * split by expert_offsets (device int32 [E+1], non-decreasing, [0] == 0,
 * [E] == T); rows [off[e], off[e+1]) take the symmetric scaled GEMM above
 * with Wq[e] (int8 [E,N,K], dense) and s_w[e] (float [E,N]) and bias[e]
 * (bf16 [E,N] or NULL). The int8 MoE scheme of [SGLang] 구조도 and the int8
 * MoE method of [Kunlun] 版本.
 * row_ids (int32 [T], nullable): sorted row r reads activation row
 * xq[row_ids[r]] and scale s_x[row_ids[r]] of an xq [M_src,K] (ldx);
 * without it xq is [T,K] in sorted order, s_x is [T] and M_src is ignored.
 * out bf16 or int32 [T,N] (ldo), in sorted order. An empty expert is legal.
 * expert_offsets and row_ids live on the device and are not checked on the
 * host; the kernel clamps offsets into [0,T] and treats a row id outside
 * [0,M_src) as an all-zero row, so bad values give wrong rows, never an
 * access outside the buffers.
 * Requires K % 16 == 0, 1 <= K <= W8A8_MAX_K, xq/Wq/out 16-byte aligned,
 * ldx % 16 == 0, ldo >= N. */
w8a8_status w8a8_grouped_scaled_mm_int8(const int8_t* xq, int64_t ldx, int64_t M_src,
                                        const int32_t* row_ids,
                                        const int32_t* expert_offsets, int64_t T, int64_t E,
                                        int64_t K, int64_t N, const int8_t* Wq,
                                        const float* s_x, const float* s_w,
                                        const uint16_t* bias, void* out, int32_t out_dtype,
                                        int64_t ldo, void* stream);

/* ---------------------------------------------------------------------------
 * The W8A8 FP8 scheme of [SGLang] 핵심 코드 분석 §1-§2: E4M3 (OCP E4M3FN)
 * weights and activations; a weight scale per tensor, per output channel or
 * per 128 x 128 block; per-token (or static per-tensor) activation scales,
 * per-token groups of 128 along K on the block path. */

/* E4M3 quantisation of bf16 activations x [M,K] (ldx) to codes xq uint8
 * [M,K] (ldq):
 *   TOKEN:    s_x[t] = max|x_t| / 448                          s_x float [M]
 *   TENSOR:   s = *s_in (device scalar)                        s_x unused
 *   GROUP128: s_x[g*M + t] = max over k in [128g, 128g+128) of |x_tk| / 448
 *             (group-major, G = ceil(K/128) groups)            s_x float [G*M]
 * An all-zero row (group) gives scale 1. xq = E4M3(clamp(x / s, -448, 448)):
 * the IEEE binary32 quotient rounded to the nearest E4M3 value, ties to even;
 * the sign of a zero is kept. Requires K % 16 == 0, K <= W8A8_MAX_K, x and
 * xq 16-byte aligned, ldx % 8 == 0, ldq % 16 == 0. */
w8a8_status w8a8_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  int32_t mode, const float* s_in, uint8_t* xq, int64_t ldq,
                                  float* s_x, void* stream);

/* The W8A8 FP8 GEMM ([SGLang] 핵심 코드 분석 §2):
 *   acc[t,n] = sum_k dec(xq[t,k]) * dec(Wq[n,k])       (binary32 MFMA sums)
 *   TENSOR / CHANNEL weight scales, TOKEN / TENSOR activation scales:
 *     y = acc * s_x[t or 0] * s_w[n or 0] + bias[n]
 *   BLOCK128 weight scales s_w [ceil(N/128), G] with GROUP128 activation
 *   scales s_x [G, M] (as w8a8_quantize_act_fp8 writes them for this M):
 *     y = sum_g acc_g[t,n] * s_x[g*M + t] * s_w[(n/128)*G + g] + bias[n]
 *     (acc_g: the sum over k in group g)
 *   out[t,n] = bf16(y) (W8A8_OUT_BF16) or y (W8A8_OUT_F32).
 * xq, Wq E4M3 codes [M,K] / [N,K] (ldx, ldw); bias bf16 [N] or NULL; out
 * [M,N] (ldo). Other mode pairs return W8A8_ERR_NOT_IMPLEMENTED. Requires
 * K % 16 == 0, 1 <= K <= W8A8_MAX_K, xq/Wq/out 16-byte aligned, ldx % 16 ==
 * 0, ldw % 16 == 0. NaN codes (0x7F, 0xFF) are outside the contract. */
w8a8_status w8a8_scaled_mm_fp8(const uint8_t* xq, int64_t M, int64_t K, int64_t ldx,
                               const uint8_t* Wq, int64_t N, int64_t ldw, const float* s_x,
                               int32_t act_mode, const float* s_w, int32_t w_mode,
                               const uint16_t* bias, void* out, int32_t out_dtype, int64_t ldo,
                               void* stream);

/* Name of the kernel instance w8a8_scaled_mm_fp8 launches for an M x N x K
 * problem with the given weight-scale mode (static storage; "" if invalid). */
const char* w8a8_scaled_mm_fp8_kernel_name(int64_t M, int64_t N, int64_t K, int32_t w_mode);

/* ---------------------------------------------------------------------------
 * The int8 MoE expert block around the grouped GEMM: the int8 MoE method of
 * [Kunlun] 版本 (experts w1 / w2 / w3, with w1 and w3 fused into one w13;
 * per-token dynamic symmetric int8 activations, per-output-channel symmetric
 * int8 weights) and the w8a8 int8 MoE scheme of [SGLang] 구조도. The pages
 * give no formula for the routing, the activation or the combine; these calls
 * take the plain readings stated with each. */

/* Bytes of workspace w8a8_moe_route needs (0 for an invalid shape). */
size_t w8a8_moe_route_workspace_size(int64_t tokens, int64_t E);

/* Top-k routing and the expert sort. For each token (row of the float router
 * logits [tokens, E], row stride ldl) the topk experts with the largest
 * logits, largest first, equal logits taken in increasing expert order:
 * topk_ids int32 [tokens, topk]; topk_w float [tokens, topk] = the softmax of
 * the selected logits. The routed (token, expert) pairs sorted by expert,
 * then token: row_ids int32 [tokens*topk] (the token of each sorted row),
 * expert_offsets int32 [E+1] (where each expert's rows start; the grouped
 * GEMM's input), pos int32 [tokens, topk] (the sorted row of each pair; the
 * combine's input). The result is fully determined (no atomics decide an
 * order). workspace: 16-byte aligned, w8a8_moe_route_workspace_size bytes,
 * no state kept. 1 <= E <= 512, 1 <= topk <= min(E, 16); NaN logits are
 * outside the contract. */
w8a8_status w8a8_moe_route(const float* logits, int64_t ldl, int64_t tokens, int64_t E,
                           int32_t topk, int32_t* topk_ids, float* topk_w, int32_t* row_ids,
                           int32_t* expert_offsets, int32_t* pos, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The activated product of a fused w13 output and its per-token symmetric
 * quantisation, the w2 GEMM's input: h bf16 [T, 2*I] (ldh) holds the gate
 * (w1) columns [0, I) and the up (w3) columns [I, 2*I);
 *   a = bf16(silu(gate) * up),  silu(g) = g / (1 + exp(-g))   (binary32)
 *   s_a[t] = max|a_t| / 127,  aq = clamp(rne(a / s_a[t]), -127, 127)
 * with the rule and exact rounding of w8a8_quantize_act (W8A8_QUANT_DYN_SYM)
 * on the bf16 values a. aq int8 [T, I] (ldq), s_a float [T]; act (nullable)
 * receives a itself, bf16 [T, I] (ld_act). I % 16 == 0, I <= 16384; h, aq,
 * act 16-byte aligned, ldh % 8 == 0, ldq % 16 == 0, ld_act % 8 == 0. */
w8a8_status w8a8_silu_mul_quant(const uint16_t* h, int64_t T, int64_t I, int64_t ldh, int8_t* aq,
                                int64_t ldq, float* s_a, uint16_t* act, int64_t ld_act,
                                void* stream);

/* The weighted combine of a token's expert outputs:
 *   out[t, :] = bf16( sum_j topk_w[t, j] * y[pos[t, j], :] )
 * (binary32 fused multiply-adds in the order j = 0 .. topk-1). y bf16 [.., N]
 * (ldy) in sorted order, pos / topk_w [tokens, topk] as w8a8_moe_route
 * writes them, out bf16 [tokens, N] (ldo). pos values must lie inside y.
 * 1 <= topk <= 16, N % 8 == 0; y and out 16-byte aligned, ldy, ldo
 * multiples of 8. */
w8a8_status w8a8_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* pos,
                             const float* topk_w, int64_t tokens, int32_t topk, int64_t N,
                             uint16_t* out, int64_t ldo, void* stream);

/* Bytes of workspace w8a8_moe_block_int8 needs (0 for an invalid shape). */
size_t w8a8_moe_block_workspace_size(int64_t tokens, int64_t E, int32_t topk, int64_t H,
                                     int64_t I);

/* The whole int8 MoE expert block for bf16 tokens x [tokens, H] (ldx):
 * per-token symmetric quantisation of x; w8a8_moe_route on the logits
 * [tokens, E] (ldl); the grouped GEMM of each routed row with its expert's
 * w13 (int8 [E, 2*I, H], per-row scales s13 float [E, 2*I]) into bf16;
 * w8a8_silu_mul_quant; the grouped GEMM with w2 (int8 [E, H, I], s2 float
 * [E, H]) into bf16; w8a8_moe_combine into out bf16 [tokens, H] (ldo). The
 * results are those of the separate calls in that order. workspace:
 * 16-byte aligned, w8a8_moe_block_workspace_size bytes, holding every
 * intermediate (no state kept). H % 16 == 0, H <= W8A8_MAX_K, I % 16 == 0,
 * I <= 16384, E <= 512, topk <= min(E, 16). */
w8a8_status w8a8_moe_block_int8(const uint16_t* x, int64_t ldx, const float* logits, int64_t ldl,
                                int64_t tokens, int64_t E, int32_t topk, int64_t H, int64_t I,
                                const int8_t* w13, const float* s13, const int8_t* w2,
                                const float* s2, uint16_t* out, int64_t ldo, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Name of the kernel template instance that w8a8_scaled_mm_int8 launches
 * for an M x N x K problem (static storage; "" for an empty or invalid
 * shape). Profilers list kernels by these names; no device is touched. */
const char* w8a8_scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K);

/* Name of the kernel that w8a8_linear_dyn_sym runs for the GEMM of an
 * M x N x K problem: the fused kernel, or the one w8a8_scaled_mm_int8 runs
 * after a separate quantiser launch (static storage; "" for an empty or
 * invalid shape). No device is touched. */
const char* w8a8_linear_dyn_sym_kernel_name(int64_t M, int64_t N, int64_t K);

/* Human-readable name of a status code (static storage); any other value
 * gives "W8A8_UNKNOWN_STATUS". The code is taken as a plain integer, so a
 * value outside the enumeration is well defined. */
const char* w8a8_status_string(int32_t status);

/* Message of the last failed call on this host thread ("" if none). */
const char* w8a8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
