"""GPU parity of w8a8_scaled_mm_int8: the corrected int32 accumulator
bit-exact (W8A8_OUT_I32) and the bf16 output within 1e-2 relative, on the
decode (M <= 64) and the MFMA tile paths, with ragged M, N and K, every
zero-point mode, per-token / per-tensor scales and bias."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed=0, full_range=True):
    rng = synth.rng_for(901, M, K, N, seed)
    lo = -128 if full_range else -127
    return dict(
        xq=rng.integers(lo, 128, (M, K), dtype=np.int8),
        w=rng.integers(lo, 128, (N, K), dtype=np.int8),
        sx=rng.uniform(1e-3, 5e-2, M).astype(np.float32),
        sw=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
        zp=rng.integers(-128, 128, M).astype(np.int32),
        bias=synth.bias_bits(rng, N),
        zin=int(rng.integers(-128, 128)),
    )


def _run(d, azp, per_token=True, per_channel=True, bias=False, out_dtype=W.OUT_BF16, ldo=None):
    M, K = d["xq"].shape
    N = d["w"].shape[0]
    note(f"scaled_mm M={M} K={K} N={N} azp={azp} pt={per_token} pc={per_channel} bias={bias} out={out_dtype}")
    xq, w = to_dev(d["xq"]), to_dev(d["w"])
    sx = to_dev(d["sx"] if per_token else d["sx"][:1])
    sw = to_dev(d["sw"] if per_channel else d["sw"][:1])
    zp = colsum = None
    if azp == W.AZP_PER_TOKEN:
        zp = to_dev(d["zp"])
        colsum = to_dev(O.colsum(d["w"]))
    elif azp == W.AZP_STATIC:
        colsum = to_dev(O.azp_adj_static(d["w"], d["zin"]))
    b = to_dev(d["bias"]) if bias else None
    out = None
    if ldo is not None:
        dt = torch.bfloat16 if out_dtype == W.OUT_BF16 else torch.int32
        out = torch.zeros((M, ldo), dtype=dt, device="cuda:0")[:, :N]
    got = W.scaled_mm_int8(xq, w, sx, sw, zp=zp, colsum=colsum, azp_mode=azp, bias=b,
                           out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    acc = O.int_gemm(d["xq"], d["w"])
    if azp == W.AZP_PER_TOKEN:
        c = O.corrected_acc(acc, zp=d["zp"], col_sum=O.colsum(d["w"]))
    elif azp == W.AZP_STATIC:
        c = O.corrected_acc(acc, azp_adj=O.azp_adj_static(d["w"], d["zin"]))
    else:
        c = acc
    if out_dtype == W.OUT_I32:
        assert_equal(host(got), c.astype(np.int32), "int32 accumulator")
    else:
        want = O.epilogue_bf16(c, d["sx"] if per_token else d["sx"][0],
                               d["sw"] if per_channel else d["sw"][0], d["bias"] if bias else None)
        assert_bf16_close(bf16_bits(got), want)


SHAPES = [(1, 256, 512), (7, 272, 520), (16, 256, 512), (33, 1040, 100), (64, 4096, 96),
          (65, 272, 130), (128, 512, 256), (200, 1296, 333), (257, 4112, 129), (1, 64, 1), (3, 16, 17)]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("azp", [W.AZP_NONE, W.AZP_PER_TOKEN, W.AZP_STATIC])
def test_i32_exact(M, K, N, azp):
    _run(_inputs(M, K, N), azp, out_dtype=W.OUT_I32)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_bf16_epilogue_variants(M, K, N):
    d = _inputs(M, K, N, seed=1)
    _run(d, W.AZP_NONE, bias=True)
    _run(d, W.AZP_PER_TOKEN, per_channel=False)
    _run(d, W.AZP_STATIC, per_token=False, bias=True)


def test_strided_output():
    d = _inputs(70, 512, 200, seed=2)
    _run(d, W.AZP_PER_TOKEN, ldo=264, out_dtype=W.OUT_I32)
    _run(d, W.AZP_NONE, ldo=208, bias=True)
    d = _inputs(9, 512, 200, seed=3)
    _run(d, W.AZP_NONE, ldo=264, out_dtype=W.OUT_I32)


@pytest.mark.parametrize("M,K,N,ldo", [(300, 256, 520, 600), (2100, 384, 2100, 2164), (2300, 640, 6100, 6144)])
def test_strided_output_tiles(M, K, N, ldo):
    """The MFMA tile path writing into a wider output (row stride ldo > N):
    every 128 x 128, 256 x 128 and 256 x 256 store form, columns past N
    left alone."""
    assert W.scaled_mm_kernel_name(M, N, K).startswith("gemm_i8_dma_kernel")
    d = _inputs(M, K, N, seed=ldo)
    _run(d, W.AZP_PER_TOKEN, ldo=ldo, out_dtype=W.OUT_I32)
    _run(d, W.AZP_NONE, ldo=ldo, bias=True)
    full = torch.full((M, ldo), -7, dtype=torch.int32, device="cuda:0")
    note(f"strided tile output padding M={M} K={K} N={N} ldo={ldo}")
    W.scaled_mm_int8(to_dev(d["xq"]), to_dev(d["w"]), to_dev(d["sx"]), to_dev(d["sw"]), out_dtype=W.OUT_I32,
                     out=full[:, :N])
    torch.cuda.synchronize()
    f = host(full)
    assert np.all(f[:, N:] == -7), "columns past N were written"
    assert_equal(f[:, :N], O.int_gemm(d["xq"], d["w"]).astype(np.int32), "strided int32")


def test_extreme_values_exact():
    """All -128 against all -128 over K = 14336: the largest sums, still exact."""
    M, K, N = 70, 14336, 40
    d = _inputs(M, K, N, seed=4)
    d["xq"][:] = -128
    d["w"][:] = -128
    d["w"][1::2] = 127
    _run(d, W.AZP_NONE, out_dtype=W.OUT_I32)
    d["xq"] = d["xq"][:5].copy()
    d["sx"], d["zp"] = d["sx"][:5], d["zp"][:5]
    _run(d, W.AZP_PER_TOKEN, out_dtype=W.OUT_I32)


@pytest.mark.parametrize("M,N", [(130, 64), (260, 520)])
def test_tile_extreme_zero_point_product(M, N):
    """The MFMA tile path's per-token correction zp * colsum at the top of its
    range: K = 65536 codes of -128, weight rows of -128 (colsum = -2^23) and
    of 127, zero points 127 and -128; every corrected sum fits int32 and must
    come out exact."""
    K = 65536
    d = _inputs(M, K, N, seed=6)
    d["xq"][:] = -128
    d["w"][0::2] = -128
    d["w"][1::2] = 127
    d["zp"][0::2] = 127
    d["zp"][1::2] = -128
    assert W.scaled_mm_kernel_name(M, N, K).startswith("gemm_i8_dma_kernel")
    _run(d, W.AZP_PER_TOKEN, out_dtype=W.OUT_I32)
    _run(d, W.AZP_PER_TOKEN, bias=True)


def test_deterministic_repeat():
    d = _inputs(64, 4096, 1000, seed=5)
    xq, w = to_dev(d["xq"]), to_dev(d["w"])
    sx, sw = to_dev(d["sx"]), to_dev(d["sw"])
    a = W.scaled_mm_int8(xq, w, sx, sw, out_dtype=W.OUT_I32)
    b = W.scaled_mm_int8(xq, w, sx, sw, out_dtype=W.OUT_I32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_empty():
    xq = torch.empty((0, 64), dtype=torch.int8, device="cuda:0")
    w = torch.zeros((8, 64), dtype=torch.int8, device="cuda:0")
    s = torch.ones(8, dtype=torch.float32, device="cuda:0")
    out = W.scaled_mm_int8(xq, w, s[:1], s)
    assert out.shape == (0, 8)


# Every decode (M <= 64) kernel instance, with ragged M and N, K = 128 (one
# step: three of four waves hold no K), and K not a multiple of 128.
DECODE_CASES = [
    (1, 14336, 4096, "gemv_reg_kernel<1, 1, 4, 4>"),
    (7, 128, 300, "gemv_reg_kernel<1, 1, 4, 4>"),
    (5, 4096, 16400, "gemv_reg_kernel<1, 1, 2, 4>"),
    (12, 4096, 28672, "gemv_shared_kernel<1, 4, true, 4>"),  # M >= 12, N > 8192
    (8, 1024, 9000, "gemv_reg_kernel<1, 1, 2, 4>"),          # 563 row groups: 2 waves
    (16, 640, 14000, "gemv_shared_kernel<1, 4, true, 4>"),   # ragged N
    (1, 4096, 4096, "gemv_reg_kernel<1, 1, 8, 2>"),
    (5, 2048, 5000, "gemv_reg_kernel<1, 2, 8, 2>"),
    (32, 1024, 200, "gemv_reg_kernel<2, 1, 4, 4>"),
    (32, 2048, 4096, "gemv_reg_kernel<2, 1, 8, 1>"),
    (17, 6144, 4100, "gemv_reg_kernel<2, 2, 4, 4>"),
    (17, 4096, 4100, "gemv_reg_kernel<2, 2, 8, 1>"),
    (48, 4096, 1000, "gemv_reg_kernel<3, 1, 4, 4>"),
    (48, 1024, 4090, "gemv_reg_kernel<3, 1, 8, 1>"),
    (33, 2048, 6000, "gemv_reg_kernel<3, 2, 4, 3>"),
    (64, 6144, 2000, "gemv_reg_kernel<4, 1, 4, 4>"),
    (64, 4096, 4096, "gemv_reg_kernel<4, 1, 8, 1>"),
    (64, 6144, 4200, "gemv_reg_kernel<4, 2, 4, 3>"),
    (60, 4096, 6130, "gemv_reg_kernel<4, 2, 8, 1>"),
    (20, 256, 16400, "gemv_shared_kernel<2, 4, true, 4>"),
    (40, 512, 16390, "gemv_shared_kernel<3, 4, true, 4>"),
    (64, 384, 16384, "gemv_shared_kernel<4, 4, true, 4>"),
    (33, 4096, 16391, "gemv_shared_kernel<3, 4, true, 4>"),
    (17, 1024, 8200, "gemv_shared_kernel<2, 4, true, 4>"),     # N just above 8192
    (64, 4096, 14336, "gemv_shared_kernel<4, 4, true, 4>"),
    (50, 8320, 9000, "gemv_shared_kernel<4, 4, true, 4>"),     # long K, N > 8192: one K range
    (40, 256, 28600, "gemv_shared_kernel<3, 4, true, 7>"),     # 256 workgroups of 112 rows, ragged
    (64, 4096, 28672, "gemv_shared_kernel<4, 4, true, 7>"),
    (64, 14336, 4096, "gemv_shared_kernel<4, 4, false, 4>"),
    (48, 8192, 1000, "gemv_shared_kernel<3, 4, false, 4>"),
    (17, 8192, 100, "gemv_shared_kernel<2, 4, false, 4>"),
    (30, 8320, 300, "gemv_shared_kernel<2, 4, false, 4>"),
    (65, 14336, 4096, "gemv_shared_kernel<5, 4, false, 4>"),   # M = 65 - 128: K ranges
    (96, 2048, 300, "gemv_shared_kernel<6, 4, false, 4>"),
    (112, 8192, 2048, "gemv_shared_kernel<7, 4, false, 4>"),
    (128, 2048, 1000, "gemv_shared_kernel<8, 4, false, 4>"),
    (128, 4096, 8200, "gemm_i8_dma_kernel<128, 128, 128, 10, false>"),  # N > 8192: MFMA tiles
    (100, 1024, 600, "gemm_i8_dma_kernel<128, 128, 128, 10, false>"),   # ranges too short
    (3, 272, 64, "gemv_i8_kernel<1, 2, 4, 8>"),
    (64, 4112, 200, "gemv_i8_kernel<4, 2, 4, 8>"),
]


@pytest.mark.parametrize("M,K,N,kernel", DECODE_CASES)
def test_decode_paths(M, K, N, kernel):
    """Each decode kernel instance: the launch table picks it, its int32
    product is exact, and a bf16 call with per-token AZP and bias matches the
    oracle's epilogue."""
    assert W.scaled_mm_kernel_name(M, N, K) == kernel
    d = _inputs(M, K, N, seed=M * 7 + N)
    note(f"decode path M={M} K={K} N={N} kernel={kernel}")
    got = W.scaled_mm_int8(to_dev(d["xq"]), to_dev(d["w"]), to_dev(d["sx"]), to_dev(d["sw"]),
                           out_dtype=W.OUT_I32)
    torch.cuda.synchronize()
    assert_equal(host(got), O.int_gemm(d["xq"], d["w"]).astype(np.int32), "decode int32")
    _run(d, W.AZP_PER_TOKEN, bias=True)


@pytest.mark.parametrize("M,K,N", [(64, 14336, 4096), (48, 8192, 1000), (96, 14336, 4096)])
def test_decode_split_without_workspace(M, K, N):
    """Without a workspace (or with one too small) a split shape runs unsplit,
    with the same exact result."""
    d = _inputs(M, K, N, seed=40)
    xq, w, sx, sw = to_dev(d["xq"]), to_dev(d["w"]), to_dev(d["sx"]), to_dev(d["sw"])
    ref = O.int_gemm(d["xq"], d["w"]).astype(np.int32)
    small = torch.empty(W.scaled_mm_workspace_size(M, N, K) - 16, dtype=torch.uint8, device="cuda:0")
    for ws in (False, small):
        got = W.scaled_mm_int8(xq, w, sx, sw, out_dtype=W.OUT_I32, workspace=ws)
        torch.cuda.synchronize()
        assert_equal(host(got), ref, "unsplit int32")


def test_decode_shape_sequence():
    """The decode shapes back to back, twice, the split ones sharing one
    workspace: exact every time (no state is carried between calls)."""
    ws = torch.empty(max(W.scaled_mm_workspace_size(M, N, K) for (M, K, N, _) in DECODE_CASES),
                     dtype=torch.uint8, device="cuda:0")
    for rep in range(2):
        for i, (M, K, N, _) in enumerate(DECODE_CASES):
            d = _inputs(M, K, N, seed=10 + i)
            note(f"decode sequence rep={rep} M={M} K={K} N={N}")
            got = W.scaled_mm_int8(to_dev(d["xq"]), to_dev(d["w"]), to_dev(d["sx"]), to_dev(d["sw"]),
                                   out_dtype=W.OUT_I32, workspace=ws)
            torch.cuda.synchronize()
            assert_equal(host(got), O.int_gemm(d["xq"], d["w"]).astype(np.int32), "decode int32")


# Every (tile, K step) variant of the MFMA path, with ragged M, N and a K that
# selects the 128-byte, the 64-byte or the zero-filled register-staged K loop.
# The shapes are chosen so that the tile-size heuristic lands on each tile
# (256 x 192 has no 64-byte variant: the heuristic passes it over there).
PATH_CASES = [
    (2300, 640, 6100, "gemm_i8_dma_kernel<256, 256, 128, 5, false>"),
    (2300, 576, 6100, "gemm_i8_dma_kernel<256, 256, 64, 10, false>"),
    (2300, 592, 6100, "gemm_i8_kernel<256, 256, false>"),
    (1800, 256, 5900, "gemm_i8_dma_kernel<256, 192, 128, 5, false>"),
    (1800, 320, 5900, "gemm_i8_dma_kernel<256, 256, 64, 10, false>"),
    (1800, 272, 5900, "gemm_i8_kernel<256, 192, false>"),
    (2100, 384, 2100, "gemm_i8_dma_kernel<256, 128, 128, 6, false>"),
    (2100, 320, 2100, "gemm_i8_dma_kernel<256, 128, 64, 10, false>"),
    (2100, 336, 2100, "gemm_i8_kernel<256, 128, false>"),
    (300, 1152, 520, "gemm_i8_dma_kernel<128, 128, 128, 10, false>"),
    (130, 192, 260, "gemm_i8_dma_kernel<128, 128, 64, 10, false>"),
    (130, 208, 260, "gemm_i8_kernel<128, 128, false>"),
]


@pytest.mark.parametrize("M,K,N,kernel", PATH_CASES)
def test_every_tile_path(M, K, N, kernel):
    assert W.scaled_mm_kernel_name(M, N, K) == kernel
    d = _inputs(M, K, N, seed=7)
    _run(d, W.AZP_PER_TOKEN, out_dtype=W.OUT_I32)
    _run(d, W.AZP_NONE, bias=True)
