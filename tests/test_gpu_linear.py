"""GPU parity of w8a8_linear_dyn_sym, the per-token symmetric quantiser and
the scaled GEMM in one call: the codes and scales it returns bit-exact
against the oracle's quantiser, the bf16 output bit-identical to the two
separate calls and within 1e-2 relative of the oracle, on the fused
single-kernel shapes (M <= 2, N <= 4096, K % 128 == 0, M * K <= 16384;
both launch shapes of it) and on shapes that take the two launches."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu

# (M, K, N, kernel of the GEMM)
CASES = [
    (1, 4096, 4096, "gemv_fused_kernel<1, 8, 2>"),
    (2, 4096, 4096, "gemv_fused_kernel<1, 8, 2>"),
    (1, 14336, 4096, "gemv_fused_kernel<1, 4, 4>"),
    (2, 1024, 300, "gemv_fused_kernel<1, 4, 4>"),     # ragged N
    (2, 128, 40, "gemv_fused_kernel<1, 4, 4>"),       # one K step: three waves have none
    (1, 256, 4090, "gemv_fused_kernel<1, 8, 2>"),     # two K steps over 8 waves, ragged N
    (2, 8192, 4096, "gemv_fused_kernel<1, 4, 4>"),    # M * K at the limit
    (1, 16384, 2048, "gemv_fused_kernel<1, 4, 4>"),   # K at the limit
    (1, 4096, 6144, "gemv_reg_kernel<1, 2, 8, 2>"),   # N > 4096: two launches
    (1, 4096, 28672, "gemv_reg_kernel<1, 1, 2, 4>"),
    (3, 1024, 300, "gemv_reg_kernel<1, 1, 4, 4>"),    # M > 2
    (4, 4096, 4100, "gemv_reg_kernel<1, 2, 8, 2>"),
    (2, 14336, 4096, "gemv_reg_kernel<1, 1, 4, 4>"),  # M * K > 16384
    (1, 4112, 300, "gemv_i8_kernel<1, 2, 4, 8>"),     # K % 128 != 0
    (64, 4096, 4096, "gemv_reg_kernel<4, 1, 8, 1>"),
    (80, 512, 256, "gemm_i8_dma_kernel<128, 128, 128, 10, false>"),  # the MFMA tile path
    (96, 2048, 300, "gemv_shared_kernel<6, 4, false, 4>"),   # M = 65 - 128: K ranges
    (128, 4096, 4096, "gemv_shared_kernel<8, 4, false, 4>"),
]


def _check(M, K, N, x_bits, w, s_w, bias):
    xd, wd, swd = to_dev(x_bits), to_dev(w), to_dev(s_w)
    bd = to_dev(bias) if bias is not None else None
    out, xq, sx = W.linear_dyn_sym(xd, wd, swd, bias=bd)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_dyn_sym(x_bits)
    assert_equal(host(xq), q_ref, "codes")
    assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), "scales")
    # the same as the two calls, bit for bit
    xq2, sx2, _ = W.quantize_act(xd, W.QUANT_DYN_SYM)
    out2 = W.scaled_mm_int8(xq2, wd, sx2, swd, bias=bd)
    torch.cuda.synchronize()
    assert_equal(bf16_bits(out), bf16_bits(out2), "fused vs separate")
    want, _ = O.scaled_mm(q_ref, w, s_ref, s_w, bias_bits=bias)
    assert_bf16_close(bf16_bits(out), want)


@pytest.mark.parametrize("M,K,N,kernel", CASES)
def test_linear_dyn_sym(M, K, N, kernel):
    assert W.linear_dyn_sym_kernel_name(M, N, K) == kernel
    d = synth.decode(M, K, N)
    note(f"linear_dyn_sym M={M} K={K} N={N} kernel={kernel}")
    _check(M, K, N, d["x"], d["w"], d["s_w"], d["bias"])


def test_linear_zero_and_outlier_rows():
    """An all-zero token row (scale 1, codes 0) next to a row with two huge
    values, a per-tensor weight scale and no bias."""
    M, K, N = 2, 2048, 1000
    rng = synth.rng_for(77, M, K, N)
    x = rng.normal(0.0, 1.0, (M, K)).astype(np.float32)
    x[0] = 0.0
    x[1, 17] = 3.0e4
    x[1, K - 1] = -2.5e4
    xb = synth.f32_to_bf16_bits(x)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    note("linear_dyn_sym zero and outlier rows")
    _check(M, K, N, xb, w, np.array([3.0e-3], np.float32), None)


def test_linear_consecutive_calls():
    """No state between calls: a wide fused call, then a smaller one."""
    for (M, K, N) in [(2, 4096, 4096), (1, 128, 16)]:
        d = synth.decode(M, K, N)
        note(f"linear_dyn_sym consecutive M={M} K={K} N={N}")
        _check(M, K, N, d["x"], d["w"], d["s_w"], d["bias"])


def test_linear_no_output_columns():
    """N == 0: only the codes and scales are written."""
    d = synth.decode(3, 1024, 8)
    xd = to_dev(d["x"])
    w = torch.empty((0, 1024), dtype=torch.int8, device="cuda:0")
    sw = torch.ones(1, dtype=torch.float32, device="cuda:0")
    note("linear_dyn_sym N=0")
    out, xq, sx = W.linear_dyn_sym(xd, w, sw)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_dyn_sym(d["x"])
    assert out.shape == (3, 0)
    assert_equal(host(xq), q_ref, "codes")
    assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), "scales")
