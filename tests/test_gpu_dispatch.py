"""GPU parity on both sides of every threshold of the decode launch table
(M <= 128), where one (M, K, N) step moves a shape to another kernel, ring
depth, wave count or K split: the int32 product bit-exact against the
oracle, and the bf16 output with per-token AZP and bias within the stated
tolerance. The kernel each side runs is named on stdout; the pairs are
chosen from the table's own conditions (token blocks of 16, row groups of 16
against 256 / 512, K steps of 128 against 40 / 64, N against 8192, the
112-row round rule), so each threshold is crossed whichever kernel it picks.
Also: the fused quantiser + GEMM limits of w8a8_linear_dyn_sym (M <= 2,
N <= 4096, M K <= 16384) against the oracle's linear forward."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth
from test_gpu_gemm import _inputs, _run

pytestmark = pytest.mark.gpu

# (M, K, N) pairs straddling one condition of the table each
BOUNDARY_PAIRS = [
    ((8, 5120, 4096), (8, 5248, 4096)),     # 40 / 41 K steps (short-K band)
    ((8, 4096, 4080), (8, 4096, 4096)),     # 255 / 256 row groups
    ((8, 4096, 8192), (8, 4096, 8208)),     # 512 / 513 row groups
    ((11, 2048, 9000), (12, 2048, 9000)),   # one token block: M >= 12 with N > 8192
    ((20, 2048, 8192), (20, 2048, 8193)),   # N > 8192: the shared kernel over the whole K
    ((32, 1024, 28672), (33, 1024, 28672)),  # 112-row workgroups from M = 33 on
    ((33, 1024, 28560), (33, 1024, 28672)),  # ... when they make whole rounds of 256
    ((20, 8064, 4096), (20, 8192, 4096)),   # 63 / 64 K steps: K ranges and the reduction
    ((64, 2048, 1000), (65, 2048, 1000)),   # 4 / 5 token blocks
    ((128, 2048, 1000), (129, 2048, 1000)),  # decode kernels (K ranges) / MFMA tiles
    ((32, 4096, 4096), (32, 4096, 4112)),   # 256 / 257 row groups at two token blocks
    ((16, 4096, 300), (16, 4112, 300)),     # K % 128: register kernel / general kernel
]
CASES = list(dict.fromkeys(s for pair in BOUNDARY_PAIRS for s in pair))


@pytest.mark.parametrize("M,K,N", CASES)
def test_decode_table_boundaries(M, K, N):
    d = _inputs(M, K, N, seed=M + 3 * N + 7 * K)
    note(f"boundary M={M} K={K} N={N} kernel={W.scaled_mm_kernel_name(M, N, K)}")
    _run(d, W.AZP_NONE, out_dtype=W.OUT_I32)
    _run(d, W.AZP_PER_TOKEN, bias=True)


@pytest.mark.parametrize("M,K,N", [(2, 4096, 4096), (3, 4096, 4096), (2, 4096, 4097), (1, 16384, 1024),
                                   (2, 8192, 1024), (2, 16384, 1024), (1, 4096, 6144)])
def test_linear_fused_limits(M, K, N):
    """linear_dyn_sym on both sides of the fused kernel's limits: codes and
    scales bit-exact, the output against the oracle's forward."""
    rng = synth.rng_for(977, M, K, N)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    bias = synth.bias_bits(rng, N)
    note(f"linear fused limits M={M} K={K} N={N} kernel={W.linear_dyn_sym_kernel_name(M, N, K)}")
    out, xq, sx = W.linear_dyn_sym(to_dev(x), to_dev(w), to_dev(sw), bias=to_dev(bias))
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_dyn_sym(x)
    assert_equal(host(xq), q_ref, "codes")
    assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), "scales")
    want, _ = O.scaled_mm(q_ref, w, s_ref, sw, bias_bits=bias)
    assert_bf16_close(bf16_bits(out), want)
