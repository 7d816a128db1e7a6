// The C ABI of libw8a8 (declared in include/w8a8.h): host-side validation,
// scheme checking, kernel dispatch and error reporting. No device memory is
// allocated at run time: buffers belong to the caller, apart from the one
// static scratch array of the no-allocation GEMM entry point below.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cmath>
#include <mutex>
#include <string>

#include "launch.h"
#include "w8a8.h"

namespace {

thread_local std::string g_last_error;

w8a8_status fail(w8a8_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w8a8_status ok() {
  g_last_error.clear();
  return W8A8_OK;
}

w8a8_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(W8A8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Per-device arch check: 0 = not yet checked, 1 = gfx950, 2 = other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

w8a8_status check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "device %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_release);
    if (st == 2)
      return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950 (MI355X)",
                  dev, prop.gcnArchName);
  }
  if (st == 2) return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950 (MI355X)", dev);
  return W8A8_OK;
}

w8a8_status check_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  return check_device(dev);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The scratch buffer of w8a8_scaled_mm_int8_noalloc: the decode GEMM's split-K
// partial tiles, in a device array the library owns (one copy per GPU, kept
// until the process ends). Host code never uses the array's name as an
// address: each device's copy is looked up once with hipGetSymbolAddress and
// that pointer is what the kernels receive. The split kernels write every
// partial they later read, so nothing in it needs to start at zero.
static __device__ __align__(256) uint8_t scratch[W8A8_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `dev`'s copy of the scratch array, looked up with that
// device current the first time it is asked for.
w8a8_status scratch_for(int dev, void** out) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return hip_status(e, "hipGetDevice");
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
      const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return hip_status(e, "hipSetDevice");
      if (eg != hipSuccess) return hip_status(eg, "hipGetSymbolAddress(scratch)");
      if (p == nullptr) return fail(W8A8_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return W8A8_OK;
}

#define W8A8_REQUIRE(cond, ...) \
  do {                          \
    if (!(cond)) return fail(W8A8_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

w8a8_status check_k(int64_t K) {
  W8A8_REQUIRE(K >= 1 && K <= W8A8_MAX_K, "K=%lld outside [1, %d]", (long long)K, W8A8_MAX_K);
  W8A8_REQUIRE(K % 16 == 0, "K=%lld is not a multiple of 16", (long long)K);
  return W8A8_OK;
}

// Sizes stay below 2^26 so that every launch's workgroup count times its
// workgroup size fits the 32-bit grid of the dispatch packet.
constexpr int64_t kMaxDim = int64_t(1) << 26;

w8a8_status check_dim(int64_t v, const char* name) {
  W8A8_REQUIRE(v >= 0 && v < kMaxDim, "%s=%lld outside [0, 2^26)", name, (long long)v);
  return W8A8_OK;
}

// Output tiles of the 128x128 MFMA GEMM (grouped: plus one partial tile per expert).
w8a8_status check_tiles(int64_t rows, int64_t extra, int64_t N) {
  const int64_t t = ((rows + 127) / 128 + extra) * ((N + 127) / 128);
  W8A8_REQUIRE(t < (int64_t(1) << 24), "problem needs %lld output tiles (limit 2^24)", (long long)t);
  return W8A8_OK;
}

}  // namespace

extern "C" {

w8a8_status w8a8_init(int device) {
  w8a8_status st = check_device(device);
  if (st != W8A8_OK) return st;
  void* p = nullptr;
  st = scratch_for(device, &p);  // the no-allocation entry point's buffer on this GPU
  return st == W8A8_OK ? ok() : st;
}

w8a8_status w8a8_check_scheme(const w8a8_scheme* s, int32_t* quant_mode, int32_t* is_channelwise) {
  W8A8_REQUIRE(s != nullptr, "scheme is NULL");
  std::string bad;
  auto note = [&](const char* what, int v) {
    char b[96];
    std::snprintf(b, sizeof b, "%s%s=%d", bad.empty() ? "" : ", ", what, v);
    bad += b;
  };
  if (s->weight_bits != 8) note("weight_bits", s->weight_bits);
  if (s->input_bits != 8) note("input_bits", s->input_bits);
  if (s->weight_strategy != W8A8_STRATEGY_TENSOR && s->weight_strategy != W8A8_STRATEGY_CHANNEL)
    note("weight_strategy", s->weight_strategy);
  if (s->weight_symmetric != 1) note("weight_symmetric", s->weight_symmetric);
  if (s->weight_dynamic != 0) note("weight_dynamic", s->weight_dynamic);
  if (s->input_symmetric != 0 && s->input_symmetric != 1) note("input_symmetric", s->input_symmetric);
  const bool static_tensor = s->input_strategy == W8A8_STRATEGY_TENSOR && s->input_dynamic == 0;
  const bool dynamic_token = s->input_strategy == W8A8_STRATEGY_TOKEN && s->input_dynamic == 1;
  if (!static_tensor && !dynamic_token) {
    note("input_strategy", s->input_strategy);
    note("input_dynamic", s->input_dynamic);
  }
  if (!bad.empty())
    return fail(W8A8_ERR_NOT_IMPLEMENTED,
                "no W8A8 INT8 scheme matches (8-bit static symmetric tensor/channel weights with "
                "static per-tensor or dynamic per-token 8-bit input): %s",
                bad.c_str());
  if (quant_mode)
    *quant_mode = dynamic_token ? (s->input_symmetric ? W8A8_QUANT_DYN_SYM : W8A8_QUANT_DYN_ASYM)
                                : (s->input_symmetric ? W8A8_QUANT_STATIC_SYM : W8A8_QUANT_STATIC_ASYM);
  if (is_channelwise) *is_channelwise = s->weight_strategy == W8A8_STRATEGY_CHANNEL;
  return ok();
}

w8a8_status w8a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int32_t mode,
                              const float* s_in, const int32_t* zp_in, int8_t* xq, int64_t ldq,
                              float* s_x, int32_t* zp, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(mode >= W8A8_QUANT_DYN_SYM && mode <= W8A8_QUANT_STATIC_ASYM, "unknown mode %d", mode);
  if (M == 0) return ok();
  W8A8_REQUIRE(x && xq, "x and xq must not be NULL");
  W8A8_REQUIRE(aligned16(x) && aligned16(xq), "x and xq must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 8 == 0, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  W8A8_REQUIRE(ldq >= K && ldq % 16 == 0, "ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
  if (mode == W8A8_QUANT_DYN_SYM || mode == W8A8_QUANT_DYN_ASYM)
    W8A8_REQUIRE(s_x != nullptr, "s_x must not be NULL in a dynamic mode");
  if (mode == W8A8_QUANT_DYN_ASYM) W8A8_REQUIRE(zp != nullptr, "zp must not be NULL in DYN_ASYM");
  if (mode == W8A8_QUANT_STATIC_SYM || mode == W8A8_QUANT_STATIC_ASYM)
    W8A8_REQUIRE(s_in != nullptr, "s_in must not be NULL in a static mode");
  if (mode == W8A8_QUANT_STATIC_ASYM) W8A8_REQUIRE(zp_in != nullptr, "zp_in must not be NULL in STATIC_ASYM");
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_quantize_act(x, M, K, ldx, mode, s_in, zp_in, xq, ldq, s_x, zp,
                                              static_cast<hipStream_t>(stream)),
                    "quantize_act launch");
}

w8a8_status w8a8_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                               float eps, uint16_t* residual, int64_t ldr, uint16_t* y, int64_t ldy, int8_t* xq,
                               int64_t ldq, float* s_x, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(std::isfinite(eps) && eps > 0.0f, "eps=%g must be finite and > 0", (double)eps);
  if (M == 0) return ok();
  W8A8_REQUIRE(x && gamma && xq && s_x, "x, gamma, xq and s_x must not be NULL");
  W8A8_REQUIRE(aligned16(x) && aligned16(gamma) && aligned16(xq) && (residual == nullptr || aligned16(residual)) &&
                   (y == nullptr || aligned16(y)),
               "x, gamma, xq, residual and y must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 8 == 0, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  W8A8_REQUIRE(ldq >= K && ldq % 16 == 0, "ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
  if (residual) W8A8_REQUIRE(ldr >= K && ldr % 8 == 0, "ldr=%lld must be >= K and a multiple of 8", (long long)ldr);
  if (y) W8A8_REQUIRE(ldy >= K && ldy % 8 == 0, "ldy=%lld must be >= K and a multiple of 8", (long long)ldy);
  W8A8_REQUIRE(y == nullptr || y != residual, "y and residual must be different buffers (y may be x)");
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_rmsnorm_quant(x, M, K, ldx, gamma, eps, residual, ldr, y, ldy, xq, ldq, s_x,
                                               static_cast<hipStream_t>(stream)),
                    "rmsnorm_quant launch");
}

w8a8_status w8a8_prepare_colsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw,
                                const int32_t* zp_in, int32_t* out, void* stream) {
  w8a8_status st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  if (N == 0) return ok();
  W8A8_REQUIRE(W && out, "W and out must not be NULL");
  W8A8_REQUIRE(aligned16(W), "W must be 16-byte aligned");
  W8A8_REQUIRE(ldw >= K && ldw % 16 == 0, "ldw=%lld must be >= K and a multiple of 16", (long long)ldw);
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_colsum(W, N, K, ldw, zp_in, out, static_cast<hipStream_t>(stream)),
                    "colsum launch");
}

w8a8_status w8a8_prepare_requant_max(int8_t* W, int64_t N, int64_t K, int64_t ldw,
                                     const float* part_scales, const int64_t* logical_widths,
                                     int32_t P, float* s_max, int32_t* err_flag, void* stream) {
  w8a8_status st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(P >= 1 && P <= W8A8_MAX_PARTITIONS, "P=%d outside [1, %d]", P, W8A8_MAX_PARTITIONS);
  W8A8_REQUIRE(part_scales && logical_widths && s_max, "part_scales, logical_widths and s_max must not be NULL");
  w8a8::RequantParts parts{};
  parts.P = P;
  int64_t sum = 0;
  for (int p = 0; p < P; ++p) {
    W8A8_REQUIRE(logical_widths[p] >= 0, "logical_widths[%d]=%lld is negative", p, (long long)logical_widths[p]);
    parts.row_start[p] = sum;
    sum += logical_widths[p];
  }
  parts.row_start[P] = sum;
  W8A8_REQUIRE(sum == N, "logical widths sum to %lld, not N=%lld", (long long)sum, (long long)N);
  W8A8_REQUIRE(N * (K / 16) < (int64_t(1) << 31), "N*K=%lld too large for one launch", (long long)(N * K));
  if (N > 0) {
    W8A8_REQUIRE(W != nullptr, "W must not be NULL");
    W8A8_REQUIRE(aligned16(W), "W must be 16-byte aligned");
    W8A8_REQUIRE(ldw >= K && ldw % 16 == 0, "ldw=%lld must be >= K and a multiple of 16", (long long)ldw);
  }
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_requant_max(W, N, K, ldw, part_scales, parts, s_max, err_flag,
                                             static_cast<hipStream_t>(stream)),
                    "requant_max launch");
}

w8a8_status w8a8_prepare_expand_scales(const float* part_scales, const int64_t* logical_widths,
                                       int32_t P, int64_t N, float* s_w, int32_t* err_flag,
                                       void* stream) {
  w8a8_status st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  W8A8_REQUIRE(P >= 1 && P <= W8A8_MAX_PARTITIONS, "P=%d outside [1, %d]", P, W8A8_MAX_PARTITIONS);
  W8A8_REQUIRE(logical_widths != nullptr, "logical_widths must not be NULL");
  w8a8::RequantParts parts{};
  parts.P = P;
  int64_t sum = 0;
  for (int p = 0; p < P; ++p) {
    W8A8_REQUIRE(logical_widths[p] >= 0, "logical_widths[%d]=%lld is negative", p, (long long)logical_widths[p]);
    parts.row_start[p] = sum;
    sum += logical_widths[p];
  }
  parts.row_start[P] = sum;
  W8A8_REQUIRE(sum == N, "logical widths sum to %lld, not N=%lld", (long long)sum, (long long)N);
  if (N == 0) return ok();
  W8A8_REQUIRE(part_scales && s_w, "part_scales and s_w must not be NULL");
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_expand_scales(part_scales, parts, N, s_w, err_flag,
                                               static_cast<hipStream_t>(stream)),
                    "expand_scales launch");
}

w8a8_status w8a8_prepare_fp8_block_to_int8(const uint8_t* W8, const float* S, int64_t E, int64_t N,
                                           int64_t K, int8_t* Wq, float* s, int32_t* err_flag,
                                           void* stream) {
  w8a8_status st;
  if ((st = check_dim(E, "E")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  if (E == 0 || N == 0) return ok();
  W8A8_REQUIRE(W8 && S && Wq && s && err_flag, "W8, S, Wq, s and err_flag must not be NULL");
  W8A8_REQUIRE(aligned16(W8) && aligned16(Wq), "W8 and Wq must be 16-byte aligned");
  W8A8_REQUIRE(E * N < kMaxDim, "E*N=%lld rows exceed 2^26", (long long)(E * N));
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_fp8_block_to_int8(W8, S, E, N, K, Wq, s, err_flag,
                                                   static_cast<hipStream_t>(stream)),
                    "fp8_block_to_int8 launch");
}

size_t w8a8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || M > w8a8::kDecodeMaxM || N >= kMaxDim || K <= 0 || K > W8A8_MAX_K) return 0;
  return w8a8::decode_workspace_bytes(M, N, K);
}

static w8a8_status check_gemm_common(const int8_t* xq, int64_t ldx, const int8_t* Wq, int64_t K,
                                     const void* out, int32_t out_dtype, int64_t ldo, int64_t N) {
  W8A8_REQUIRE(xq && Wq && out, "xq, Wq and out must not be NULL");
  W8A8_REQUIRE(aligned16(xq) && aligned16(Wq) && aligned16(out), "xq, Wq and out must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 16 == 0, "ldx=%lld must be >= K and a multiple of 16", (long long)ldx);
  W8A8_REQUIRE(ldo >= N, "ldo=%lld must be >= N", (long long)ldo);
  W8A8_REQUIRE(out_dtype == W8A8_OUT_BF16 || out_dtype == W8A8_OUT_I32, "unknown out_dtype %d", out_dtype);
  return W8A8_OK;
}

// Shared body of w8a8_scaled_mm_int8 and w8a8_scaled_mm_int8_noalloc.
// noalloc: the workspace is the current device's static scratch array.
static w8a8_status scaled_mm_impl(const int8_t* xq, int64_t M, int64_t K, int64_t ldx, const int8_t* Wq,
                                  int64_t N, int64_t ldw, const float* s_x, int32_t s_x_per_token,
                                  const float* s_w, int32_t s_w_per_channel, const int32_t* zp,
                                  const int32_t* colsum, int32_t azp_mode, const uint16_t* bias, void* out,
                                  int32_t out_dtype, int64_t ldo, void* workspace, size_t workspace_bytes,
                                  bool noalloc, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(azp_mode >= W8A8_AZP_NONE && azp_mode <= W8A8_AZP_STATIC, "unknown azp_mode %d", azp_mode);
  if (M == 0 || N == 0) return ok();
  if ((st = check_gemm_common(xq, ldx, Wq, K, out, out_dtype, ldo, N)) != W8A8_OK) return st;
  W8A8_REQUIRE(ldw >= K && ldw % 16 == 0, "ldw=%lld must be >= K and a multiple of 16", (long long)ldw);
  W8A8_REQUIRE(s_x && s_w, "s_x and s_w must not be NULL");
  if (azp_mode == W8A8_AZP_PER_TOKEN) W8A8_REQUIRE(zp && colsum, "AZP_PER_TOKEN needs zp and colsum");
  if (azp_mode == W8A8_AZP_STATIC) W8A8_REQUIRE(colsum, "AZP_STATIC needs azp_adj (passed as colsum)");
  if ((st = check_tiles(M, 0, N)) != W8A8_OK) return st;
  W8A8_REQUIRE(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  if ((st = check_current_device()) != W8A8_OK) return st;
  if (noalloc) {
    const size_t need = M <= w8a8::kDecodeMaxM ? w8a8::decode_workspace_bytes(M, N, K) : 0;
    W8A8_REQUIRE(need <= W8A8_NOALLOC_SCRATCH_BYTES,
                 "shape %lld x %lld x %lld needs %zu bytes of scratch; the static buffer holds %d",
                 (long long)M, (long long)N, (long long)K, need, W8A8_NOALLOC_SCRATCH_BYTES);
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if ((st = scratch_for(dev, &workspace)) != W8A8_OK) return st;
    workspace_bytes = W8A8_NOALLOC_SCRATCH_BYTES;
  }
  w8a8::GemmArgs a{};
  a.A = xq;
  a.lda = ldx;
  a.B = Wq;
  a.ldb = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.s_x = s_x;
  a.sx_per_token = s_x_per_token != 0;
  a.s_w = s_w;
  a.sw_per_channel = s_w_per_channel != 0;
  a.zp = zp;
  a.colsum = colsum;
  a.azp_mode = azp_mode;
  a.bias = bias;
  a.out = out;
  a.out_i32 = out_dtype == W8A8_OUT_I32;
  a.ldo = ldo;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = (M <= w8a8::kDecodeMaxM)
                           ? w8a8::launch_decode_mm(a, workspace, workspace_bytes, s)
                           : w8a8::launch_scaled_mm(a, s);
  return hip_status(e, "scaled_mm launch");
}

w8a8_status w8a8_scaled_mm_int8(const int8_t* xq, int64_t M, int64_t K, int64_t ldx, const int8_t* Wq,
                                int64_t N, int64_t ldw, const float* s_x, int32_t s_x_per_token,
                                const float* s_w, int32_t s_w_per_channel, const int32_t* zp,
                                const int32_t* colsum, int32_t azp_mode, const uint16_t* bias, void* out,
                                int32_t out_dtype, int64_t ldo, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return scaled_mm_impl(xq, M, K, ldx, Wq, N, ldw, s_x, s_x_per_token, s_w, s_w_per_channel, zp, colsum,
                        azp_mode, bias, out, out_dtype, ldo, workspace, workspace_bytes, false, stream);
}

w8a8_status w8a8_scaled_mm_int8_noalloc(const int8_t* xq, int64_t M, int64_t K, int64_t ldx,
                                        const int8_t* Wq, int64_t N, int64_t ldw, const float* s_x,
                                        int32_t s_x_per_token, const float* s_w, int32_t s_w_per_channel,
                                        const int32_t* zp, const int32_t* colsum, int32_t azp_mode,
                                        const uint16_t* bias, void* out, int32_t out_dtype, int64_t ldo,
                                        void* stream) {
  return scaled_mm_impl(xq, M, K, ldx, Wq, N, ldw, s_x, s_x_per_token, s_w, s_w_per_channel, zp, colsum,
                        azp_mode, bias, out, out_dtype, ldo, nullptr, 0, true, stream);
}

w8a8_status w8a8_linear_dyn_sym(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* Wq,
                                int64_t N, int64_t ldw, const float* s_w, int32_t s_w_per_channel,
                                const uint16_t* bias, uint16_t* out, int64_t ldo, int8_t* xq, int64_t ldq,
                                float* s_x, void* workspace, size_t workspace_bytes, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  if (M == 0) return ok();
  W8A8_REQUIRE(x && xq && s_x, "x, xq and s_x must not be NULL");
  W8A8_REQUIRE(aligned16(x) && aligned16(xq), "x and xq must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 8 == 0, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  W8A8_REQUIRE(ldq >= K && ldq % 16 == 0, "ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
  if (N > 0) {
    if ((st = check_gemm_common(xq, ldq, Wq, K, out, W8A8_OUT_BF16, ldo, N)) != W8A8_OK) return st;
    W8A8_REQUIRE(ldw >= K && ldw % 16 == 0, "ldw=%lld must be >= K and a multiple of 16", (long long)ldw);
    W8A8_REQUIRE(s_w != nullptr, "s_w must not be NULL");
    if ((st = check_tiles(M, 0, N)) != W8A8_OK) return st;
  }
  W8A8_REQUIRE(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  if ((st = check_current_device()) != W8A8_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  w8a8::GemmArgs a{};
  a.A = xq;
  a.lda = ldq;
  a.B = Wq;
  a.ldb = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.s_x = s_x;
  a.sx_per_token = 1;
  a.s_w = s_w;
  a.sw_per_channel = s_w_per_channel != 0;
  a.azp_mode = W8A8_AZP_NONE;
  a.bias = bias;
  a.out = out;
  a.out_i32 = 0;
  a.ldo = ldo;
  if (w8a8::fused_linear_fits(M, N, K))
    return hip_status(w8a8::launch_fused_linear(a, x, ldx, xq, ldq, s_x, s), "fused linear launch");
  // otherwise the two launches, in order on the stream
  hipError_t e = w8a8::launch_quantize_act(x, M, K, ldx, W8A8_QUANT_DYN_SYM, nullptr, nullptr, xq, ldq, s_x,
                                           nullptr, s);
  if (e != hipSuccess || N == 0) return hip_status(e, "quantize_act launch");
  e = (M <= w8a8::kDecodeMaxM) ? w8a8::launch_decode_mm(a, workspace, workspace_bytes, s)
                               : w8a8::launch_scaled_mm(a, s);
  return hip_status(e, "scaled_mm launch");
}

const char* w8a8_linear_dyn_sym_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return "";
  if (w8a8::fused_linear_fits(M, N, K)) return w8a8::fused_linear_kernel_name(M, N, K);
  return w8a8_scaled_mm_kernel_name(M, N, K);
}

w8a8_status w8a8_grouped_scaled_mm_int8(const int8_t* xq, int64_t ldx, int64_t M_src, const int32_t* row_ids,
                                        const int32_t* expert_offsets, int64_t T, int64_t E, int64_t K,
                                        int64_t N, const int8_t* Wq, const float* s_x, const float* s_w,
                                        const uint16_t* bias, void* out, int32_t out_dtype, int64_t ldo,
                                        void* stream) {
  w8a8_status st;
  if ((st = check_dim(T, "T")) != W8A8_OK) return st;
  if ((st = check_dim(E, "E")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  if (T == 0 || E == 0 || N == 0) return ok();
  if ((st = check_gemm_common(xq, ldx, Wq, K, out, out_dtype, ldo, N)) != W8A8_OK) return st;
  W8A8_REQUIRE(expert_offsets && s_x && s_w, "expert_offsets, s_x and s_w must not be NULL");
  if (row_ids) {
    if ((st = check_dim(M_src, "M_src")) != W8A8_OK) return st;
    W8A8_REQUIRE(M_src >= 1, "M_src must be >= 1 with row_ids");
  }
  if ((st = check_tiles(T, E, N)) != W8A8_OK) return st;
  if ((st = check_current_device()) != W8A8_OK) return st;
  w8a8::GemmArgs a{};
  a.A = xq;
  a.lda = ldx;
  a.B = Wq;
  a.ldb = K;
  a.M = T;
  a.N = N;
  a.K = K;
  a.s_x = s_x;
  a.sx_per_token = 1;
  a.s_w = s_w;
  a.sw_per_channel = 1;
  a.azp_mode = W8A8_AZP_NONE;
  a.bias = bias;
  a.out = out;
  a.out_i32 = out_dtype == W8A8_OUT_I32;
  a.ldo = ldo;
  a.row_ids = row_ids;
  a.expert_offsets = expert_offsets;
  a.E = E;
  a.M_src = row_ids ? M_src : T;
  return hip_status(w8a8::launch_grouped_mm(a, static_cast<hipStream_t>(stream)), "grouped_mm launch");
}

w8a8_status w8a8_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int32_t mode,
                                  const float* s_in, uint8_t* xq, int64_t ldq, float* s_x, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(mode >= W8A8_FP8_ACT_TOKEN && mode <= W8A8_FP8_ACT_GROUP128, "unknown FP8 mode %d", mode);
  if (M == 0) return ok();
  W8A8_REQUIRE(x && xq, "x and xq must not be NULL");
  W8A8_REQUIRE(aligned16(x) && aligned16(xq), "x and xq must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 8 == 0, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  W8A8_REQUIRE(ldq >= K && ldq % 16 == 0, "ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
  if (mode == W8A8_FP8_ACT_TENSOR) W8A8_REQUIRE(s_in != nullptr, "s_in must not be NULL in TENSOR mode");
  else W8A8_REQUIRE(s_x != nullptr, "s_x must not be NULL in a dynamic mode");
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_quantize_act_fp8(x, M, K, ldx, mode, s_in, xq, ldq, s_x,
                                                  static_cast<hipStream_t>(stream)),
                    "quantize_act_fp8 launch");
}

w8a8_status w8a8_scaled_mm_fp8(const uint8_t* xq, int64_t M, int64_t K, int64_t ldx, const uint8_t* Wq, int64_t N,
                               int64_t ldw, const float* s_x, int32_t act_mode, const float* s_w, int32_t w_mode,
                               const uint16_t* bias, void* out, int32_t out_dtype, int64_t ldo, void* stream) {
  w8a8_status st;
  if ((st = check_dim(M, "M")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  if ((st = check_k(K)) != W8A8_OK) return st;
  W8A8_REQUIRE(act_mode >= W8A8_FP8_ACT_TOKEN && act_mode <= W8A8_FP8_ACT_GROUP128, "unknown act_mode %d",
               act_mode);
  W8A8_REQUIRE(w_mode >= W8A8_FP8_W_TENSOR && w_mode <= W8A8_FP8_W_BLOCK128, "unknown w_mode %d", w_mode);
  const bool block = w_mode == W8A8_FP8_W_BLOCK128;
  if (block != (act_mode == W8A8_FP8_ACT_GROUP128))
    return fail(W8A8_ERR_NOT_IMPLEMENTED,
                "FP8 scales: 128x128 weight blocks go with per-token groups of 128 activations, "
                "tensor/channel weights with token/tensor activations (got w_mode=%d, act_mode=%d)",
                w_mode, act_mode);
  W8A8_REQUIRE(out_dtype == W8A8_OUT_BF16 || out_dtype == W8A8_OUT_F32, "out_dtype must be BF16 or F32");
  if (M == 0 || N == 0) return ok();
  W8A8_REQUIRE(xq && Wq && out && s_x && s_w, "xq, Wq, out, s_x and s_w must not be NULL");
  W8A8_REQUIRE(aligned16(xq) && aligned16(Wq) && aligned16(out), "xq, Wq and out must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= K && ldx % 16 == 0, "ldx=%lld must be >= K and a multiple of 16", (long long)ldx);
  W8A8_REQUIRE(ldw >= K && ldw % 16 == 0, "ldw=%lld must be >= K and a multiple of 16", (long long)ldw);
  W8A8_REQUIRE(ldo >= N, "ldo=%lld must be >= N", (long long)ldo);
  if ((st = check_tiles(M, 0, N)) != W8A8_OK) return st;
  if ((st = check_current_device()) != W8A8_OK) return st;
  w8a8::GemmArgs a{};
  a.A = reinterpret_cast<const int8_t*>(xq);
  a.lda = ldx;
  a.B = reinterpret_cast<const int8_t*>(Wq);
  a.ldb = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.s_x = s_x;
  a.sx_per_token = act_mode == W8A8_FP8_ACT_TOKEN;
  a.s_w = s_w;
  a.sw_per_channel = w_mode == W8A8_FP8_W_CHANNEL;
  a.azp_mode = W8A8_AZP_NONE;
  a.bias = bias;
  a.out = out;
  a.out_i32 = out_dtype == W8A8_OUT_F32;
  a.ldo = ldo;
  return hip_status(w8a8::launch_scaled_mm_fp8(a, block, static_cast<hipStream_t>(stream)), "scaled_mm_fp8 launch");
}

const char* w8a8_scaled_mm_fp8_kernel_name(int64_t M, int64_t N, int64_t K, int32_t w_mode) {
  if (M <= 0 || N <= 0 || K <= 0 || w_mode < W8A8_FP8_W_TENSOR || w_mode > W8A8_FP8_W_BLOCK128) return "";
  return w8a8::scaled_mm_fp8_kernel_name(M, N, K, w_mode == W8A8_FP8_W_BLOCK128);
}

}  // extern "C"

// ------------------------------------------------------------ MoE block

namespace {

constexpr int kMoeMaxExperts = 512;
constexpr int kMoeMaxTopk = 16;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t route_ws_bytes(int64_t tokens, int64_t E) {
  return align256((size_t)w8a8::moe_route_chunks(tokens) * (size_t)E * sizeof(uint64_t));
}

w8a8_status check_moe_shape(int64_t tokens, int64_t E, int32_t topk) {
  w8a8_status st;
  if ((st = check_dim(tokens, "tokens")) != W8A8_OK) return st;
  W8A8_REQUIRE(E >= 1 && E <= kMoeMaxExperts, "E=%lld outside [1, %d]", (long long)E, kMoeMaxExperts);
  W8A8_REQUIRE(topk >= 1 && topk <= kMoeMaxTopk && topk <= E, "topk=%d outside [1, min(E, %d)]", topk,
               kMoeMaxTopk);
  W8A8_REQUIRE(tokens * topk < kMaxDim, "tokens*topk=%lld routed rows exceed 2^26", (long long)(tokens * topk));
  return W8A8_OK;
}

// Where each intermediate of w8a8_moe_block_int8 sits in its workspace
// (256-byte aligned pieces; the w2 output reuses the w13 output's bytes,
// which are dead once the activated product is quantised).
struct MoeLayout {
  size_t xq, sx, ids, wts, row_ids, offsets, pos, masks, h, aq, sa, y, total;
};

MoeLayout moe_layout(int64_t tokens, int64_t E, int32_t topk, int64_t H, int64_t I) {
  MoeLayout L{};
  const size_t T = (size_t)tokens * (size_t)topk;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.xq = take((size_t)tokens * H);
  L.sx = take((size_t)tokens * 4);
  L.ids = take(T * 4);
  L.wts = take(T * 4);
  L.row_ids = take(T * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.pos = take(T * 4);
  L.masks = take(route_ws_bytes(tokens, E));
  L.aq = take(T * (size_t)I);
  L.sa = take(T * 4);
  const size_t h_bytes = T * (size_t)(2 * I) * 2, y_bytes = T * (size_t)H * 2;
  L.h = take(h_bytes > y_bytes ? h_bytes : y_bytes);
  L.y = L.h;
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t w8a8_moe_route_workspace_size(int64_t tokens, int64_t E) {
  if (tokens <= 0 || tokens >= kMaxDim || E <= 0 || E > kMoeMaxExperts) return 0;
  return route_ws_bytes(tokens, E);
}

w8a8_status w8a8_moe_route(const float* logits, int64_t ldl, int64_t tokens, int64_t E, int32_t topk,
                           int32_t* topk_ids, float* topk_w, int32_t* row_ids, int32_t* expert_offsets,
                           int32_t* pos, void* workspace, size_t workspace_bytes, void* stream) {
  w8a8_status st;
  if ((st = check_moe_shape(tokens, E, topk)) != W8A8_OK) return st;
  if (tokens == 0) return ok();
  W8A8_REQUIRE(logits && topk_ids && topk_w && row_ids && expert_offsets && pos,
               "logits, topk_ids, topk_w, row_ids, expert_offsets and pos must not be NULL");
  W8A8_REQUIRE(ldl >= E, "ldl=%lld must be >= E", (long long)ldl);
  W8A8_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= route_ws_bytes(tokens, E),
               "routing needs a 16-byte aligned workspace of %zu bytes", route_ws_bytes(tokens, E));
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_moe_route(logits, ldl, tokens, (int)E, topk, topk_ids, topk_w, row_ids,
                                           expert_offsets, pos, static_cast<uint64_t*>(workspace),
                                           static_cast<hipStream_t>(stream)),
                    "moe_route launch");
}

w8a8_status w8a8_silu_mul_quant(const uint16_t* h, int64_t T, int64_t I, int64_t ldh, int8_t* aq, int64_t ldq,
                                float* s_a, uint16_t* act, int64_t ld_act, void* stream) {
  w8a8_status st;
  if ((st = check_dim(T, "T")) != W8A8_OK) return st;
  W8A8_REQUIRE(I >= 1 && I <= 16384 && I % 16 == 0, "I=%lld must be a multiple of 16 in [16, 16384]",
               (long long)I);
  if (T == 0) return ok();
  W8A8_REQUIRE(h && aq && s_a, "h, aq and s_a must not be NULL");
  W8A8_REQUIRE(aligned16(h) && aligned16(aq) && (act == nullptr || aligned16(act)),
               "h, aq and act must be 16-byte aligned");
  W8A8_REQUIRE(ldh >= 2 * I && ldh % 8 == 0, "ldh=%lld must be >= 2*I and a multiple of 8", (long long)ldh);
  W8A8_REQUIRE(ldq >= I && ldq % 16 == 0, "ldq=%lld must be >= I and a multiple of 16", (long long)ldq);
  if (act) W8A8_REQUIRE(ld_act >= I && ld_act % 8 == 0, "ld_act=%lld must be >= I and a multiple of 8",
                        (long long)ld_act);
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_silu_mul_quant(h, T, I, ldh, aq, ldq, s_a, act, ld_act,
                                                static_cast<hipStream_t>(stream)),
                    "silu_mul_quant launch");
}

w8a8_status w8a8_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* pos, const float* topk_w,
                             int64_t tokens, int32_t topk, int64_t N, uint16_t* out, int64_t ldo, void* stream) {
  w8a8_status st;
  if ((st = check_dim(tokens, "tokens")) != W8A8_OK) return st;
  if ((st = check_dim(N, "N")) != W8A8_OK) return st;
  W8A8_REQUIRE(topk >= 1 && topk <= kMoeMaxTopk, "topk=%d outside [1, %d]", topk, kMoeMaxTopk);
  W8A8_REQUIRE(N % 8 == 0, "N=%lld must be a multiple of 8", (long long)N);
  if (tokens == 0 || N == 0) return ok();
  W8A8_REQUIRE(y && pos && topk_w && out, "y, pos, topk_w and out must not be NULL");
  W8A8_REQUIRE(aligned16(y) && aligned16(out), "y and out must be 16-byte aligned");
  W8A8_REQUIRE(ldy >= N && ldy % 8 == 0 && ldo >= N && ldo % 8 == 0,
               "ldy and ldo must be >= N and multiples of 8");
  if ((st = check_current_device()) != W8A8_OK) return st;
  return hip_status(w8a8::launch_moe_combine(y, ldy, pos, topk_w, tokens, topk, N, out, ldo,
                                             static_cast<hipStream_t>(stream)),
                    "moe_combine launch");
}

size_t w8a8_moe_block_workspace_size(int64_t tokens, int64_t E, int32_t topk, int64_t H, int64_t I) {
  if (tokens <= 0 || tokens >= kMaxDim || E <= 0 || E > kMoeMaxExperts || topk <= 0 || H <= 0 || I <= 0)
    return 0;
  return moe_layout(tokens, E, topk, H, I).total;
}

w8a8_status w8a8_moe_block_int8(const uint16_t* x, int64_t ldx, const float* logits, int64_t ldl,
                                int64_t tokens, int64_t E, int32_t topk, int64_t H, int64_t I,
                                const int8_t* w13, const float* s13, const int8_t* w2, const float* s2,
                                uint16_t* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                                void* stream) {
  w8a8_status st;
  if ((st = check_moe_shape(tokens, E, topk)) != W8A8_OK) return st;
  if ((st = check_k(H)) != W8A8_OK) return st;
  W8A8_REQUIRE(I >= 16 && I <= 16384 && I % 16 == 0, "I=%lld must be a multiple of 16 in [16, 16384]",
               (long long)I);
  if (tokens == 0) return ok();
  W8A8_REQUIRE(x && logits && w13 && s13 && w2 && s2 && out, "no array may be NULL");
  W8A8_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(out),
               "x, w13, w2 and out must be 16-byte aligned");
  W8A8_REQUIRE(ldx >= H && ldx % 8 == 0, "ldx=%lld must be >= H and a multiple of 8", (long long)ldx);
  W8A8_REQUIRE(ldl >= E, "ldl=%lld must be >= E", (long long)ldl);
  W8A8_REQUIRE(ldo >= H && ldo % 8 == 0, "ldo=%lld must be >= H and a multiple of 8", (long long)ldo);
  const int64_t T = tokens * topk;
  if ((st = check_tiles(T, E, 2 * I)) != W8A8_OK) return st;
  if ((st = check_tiles(T, E, H)) != W8A8_OK) return st;
  const MoeLayout L = moe_layout(tokens, E, topk, H, I);
  W8A8_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= L.total,
               "the block needs a 16-byte aligned workspace of %zu bytes", L.total);
  if ((st = check_current_device()) != W8A8_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = reinterpret_cast<float*>(ws + L.wts);
  int32_t* row_ids = reinterpret_cast<int32_t*>(ws + L.row_ids);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  uint64_t* masks = reinterpret_cast<uint64_t*>(ws + L.masks);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  int8_t* aq = reinterpret_cast<int8_t*>(ws + L.aq);
  float* sa = reinterpret_cast<float*>(ws + L.sa);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);

  hipError_t e = w8a8::launch_quantize_act(x, tokens, H, ldx, W8A8_QUANT_DYN_SYM, nullptr, nullptr, xq, H, sx,
                                           nullptr, s);
  if (e != hipSuccess) return hip_status(e, "quantize_act launch");
  e = w8a8::launch_moe_route(logits, ldl, tokens, (int)E, topk, ids, wts, row_ids, offsets, pos, masks, s);
  if (e != hipSuccess) return hip_status(e, "moe_route launch");
  w8a8::GemmArgs g{};
  g.A = xq;
  g.lda = H;
  g.B = w13;
  g.ldb = H;
  g.M = T;
  g.N = 2 * I;
  g.K = H;
  g.s_x = sx;
  g.sx_per_token = 1;
  g.s_w = s13;
  g.sw_per_channel = 1;
  g.azp_mode = W8A8_AZP_NONE;
  g.out = h;
  g.ldo = 2 * I;
  g.row_ids = row_ids;
  g.expert_offsets = offsets;
  g.E = E;
  g.M_src = tokens;
  if ((e = w8a8::launch_grouped_mm(g, s)) != hipSuccess) return hip_status(e, "grouped w13 launch");
  e = w8a8::launch_silu_mul_quant(h, T, I, 2 * I, aq, I, sa, nullptr, 0, s);
  if (e != hipSuccess) return hip_status(e, "silu_mul_quant launch");
  g.A = aq;
  g.lda = I;
  g.B = w2;
  g.ldb = I;
  g.N = H;
  g.K = I;
  g.s_x = sa;
  g.s_w = s2;
  g.out = y;
  g.ldo = H;
  g.row_ids = nullptr;
  g.M_src = T;
  if ((e = w8a8::launch_grouped_mm(g, s)) != hipSuccess) return hip_status(e, "grouped w2 launch");
  return hip_status(w8a8::launch_moe_combine(y, H, pos, wts, tokens, topk, H, out, ldo, s), "moe_combine launch");
}

const char* w8a8_scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return "";
  return (M <= w8a8::kDecodeMaxM) ? w8a8::decode_kernel_name(M, N, K, w8a8::decode_workspace_bytes(M, N, K)) : w8a8::scaled_mm_kernel_name(M, N, K);
}

const char* w8a8_status_string(int32_t s) {
  switch (s) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_ERR_INVALID_ARG: return "W8A8_ERR_INVALID_ARG";
    case W8A8_ERR_NOT_IMPLEMENTED: return "W8A8_ERR_NOT_IMPLEMENTED";
    case W8A8_ERR_UNSUPPORTED_DEVICE: return "W8A8_ERR_UNSUPPORTED_DEVICE";
    case W8A8_ERR_HIP: return "W8A8_ERR_HIP";
  }
  return "W8A8_UNKNOWN_STATUS";
}

const char* w8a8_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
