"""GPU parity with padded operands and outputs, through the C ABI: the row
strides of the activation codes and of the weight past K, and of the output
past N (odd ones included), on every GEMM family -- the decode kernels
(register, shared over the whole K, shared over K ranges with the reduction,
general), the fused quantiser + GEMM, the MFMA tiles (each tile size and K
step), the grouped MoE GEMM (sorted and gathered rows) and the FP8 GEMM
(ring, block-scaled ring, register-staged). The int32 products are compared
with the oracle; every bf16 / binary32 result is bit-identical to the same
call on packed tensors (whose parity the other files prove); the padding of
the output is left as it was."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_equal, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _padded(a, ld, fill):
    """A device copy of the 2-D host array a inside a [rows, ld] buffer
    filled with `fill`, as a strided view of the first columns."""
    buf = np.full((a.shape[0], ld), fill, dtype=a.dtype)
    buf[:, :a.shape[1]] = a
    return to_dev(buf)[:, :a.shape[1]]


def _out(M, N, ldo, dtype, fill):
    return torch.full((M, ldo), fill, dtype=dtype, device=DEV)[:, :N]


def _bits(t):
    return host(t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous())


def _pad_untouched(view, ldo, fill, what):
    full = host(view.as_strided((view.shape[0], ldo), (view.stride(0), 1)))
    want = np.full((view.shape[0], ldo - view.shape[1]), fill).astype(full.dtype)
    assert np.array_equal(full[:, view.shape[1]:], want), f"{what}: output padding written"


GEMM_CASES = [
    (8, 512, 300, "gemv_reg_kernel"),
    (20, 2048, 8200, "gemv_shared_kernel<2, 4, true"),
    (20, 8192, 300, "gemv_shared_kernel<2, 4, false"),
    (16, 272, 100, "gemv_i8_kernel"),
    (300, 256, 520, "gemm_i8_dma_kernel<128, 128, 128"),
    (2100, 384, 2100, "gemm_i8_dma_kernel<256, 128, 128"),
    (2300, 640, 6100, "gemm_i8_dma_kernel<256, 256, 128"),
    (2300, 576, 6100, "gemm_i8_dma_kernel<256, 256, 64"),
    (130, 208, 260, "gemm_i8_kernel<128, 128"),
]


@pytest.mark.parametrize("M,K,N,kernel", GEMM_CASES)
@pytest.mark.parametrize("ldo_pad", [3, 40])
def test_scaled_mm_padded(M, K, N, kernel, ldo_pad):
    assert W.scaled_mm_kernel_name(M, N, K).startswith(kernel)
    rng = synth.rng_for(985, M, K, N, ldo_pad)
    xq = rng.integers(-128, 128, (M, K), dtype=np.int8)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 5e-2, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    zp = rng.integers(-128, 128, M).astype(np.int32)
    bias = synth.bias_bits(rng, N)
    ldx, ldw, ldo = K + 48, K + 32, N + ldo_pad
    note(f"padded scaled_mm M={M} K={K} N={N} ldx={ldx} ldw={ldw} ldo={ldo}")
    xd, wd = _padded(xq, ldx, 77), _padded(w, ldw, -99)
    sxd, swd, zpd = to_dev(sx), to_dev(sw), to_dev(zp)
    cs = to_dev(O.colsum(w))
    # int32 with per-token AZP against the oracle
    oi = _out(M, N, ldo, torch.int32, -5)
    W.scaled_mm_int8(xd, wd, sxd, swd, zp=zpd, colsum=cs, azp_mode=W.AZP_PER_TOKEN, out_dtype=W.OUT_I32, out=oi)
    torch.cuda.synchronize()
    want = O.corrected_acc(O.int_gemm(xq, w), zp=zp, col_sum=O.colsum(w)).astype(np.int32)
    assert_equal(host(oi.contiguous()), want, "padded int32")
    _pad_untouched(oi, ldo, -5, "int32")
    # bf16 with bias: the same bits as the packed call
    ob = _out(M, N, ldo, torch.bfloat16, 0.5)
    W.scaled_mm_int8(xd, wd, sxd, swd, bias=to_dev(bias), out=ob)
    packed = W.scaled_mm_int8(to_dev(xq), to_dev(w), sxd, swd, bias=to_dev(bias))
    torch.cuda.synchronize()
    assert_equal(_bits(ob), _bits(packed), "padded bf16 against packed")
    _pad_untouched(ob.view(torch.int16), ldo, np.int16(0x3F00), "bf16")


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (2, 4096, 4096), (8, 4096, 600)])
def test_linear_dyn_sym_padded(M, K, N):
    """The fused kernel (M <= 2) and the two launches, on padded x, codes and output."""
    rng = synth.rng_for(986, M, K, N)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = to_dev(rng.uniform(1e-3, 1e-2, N).astype(np.float32))
    bias = to_dev(synth.bias_bits(rng, N))
    ldx, ldq, ldo = K + 24, K + 16, N + 5
    note(f"padded linear_dyn_sym M={M} K={K} N={N} kernel={W.linear_dyn_sym_kernel_name(M, N, K)}")
    xd = _padded(x.view(np.int16), ldx, 0).view(torch.bfloat16)
    xq = torch.full((M, ldq), 9, dtype=torch.int8, device=DEV)[:, :K]
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    out = _out(M, N, ldo, torch.bfloat16, 0.5)
    W.linear_dyn_sym(xd, to_dev(w), sw, bias=bias, out=out, xq=xq, s_x=sx)
    ref_out, ref_q, ref_s = W.linear_dyn_sym(to_dev(x), to_dev(w), sw, bias=bias)
    torch.cuda.synchronize()
    assert_equal(host(xq.contiguous()), O.quant_dyn_sym(x)[0], "codes")
    _pad_untouched(xq, ldq, 9, "codes")
    assert_equal(host(sx).view(np.uint32), host(ref_s).view(np.uint32), "scales")
    assert_equal(_bits(out), _bits(ref_out), "output against packed")
    _pad_untouched(out.view(torch.int16), ldo, np.int16(0x3F00), "output")


@pytest.mark.parametrize("gather", [False, True])
def test_grouped_padded(gather):
    E, K, N, T = 5, 384, 300, 900
    rng = synth.rng_for(987, int(gather))
    counts = np.array([0, 400, 1, 260, 239])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M_src = 350 if gather else T
    xq = rng.integers(-128, 128, (M_src, K), dtype=np.int8)
    rid = rng.integers(0, M_src, T).astype(np.int32) if gather else None
    w = rng.integers(-128, 128, (E, N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 5e-2, M_src).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, (E, N)).astype(np.float32)
    ldx, ldo = K + 64, N + 7
    note(f"padded grouped gather={gather} T={T} ldx={ldx} ldo={ldo}")
    args = dict(row_ids=None if rid is None else to_dev(rid), T=T)
    oi = _out(T, N, ldo, torch.int32, -5)
    W.grouped_scaled_mm_int8(_padded(xq, ldx, 3), to_dev(off), to_dev(w), to_dev(sx), to_dev(sw),
                             out_dtype=W.OUT_I32, out=oi, **args)
    ob = _out(T, N, ldo, torch.bfloat16, 0.5)
    W.grouped_scaled_mm_int8(_padded(xq, ldx, 3), to_dev(off), to_dev(w), to_dev(sx), to_dev(sw), out=ob, **args)
    packed = W.grouped_scaled_mm_int8(to_dev(xq), to_dev(off), to_dev(w), to_dev(sx), to_dev(sw), **args)
    torch.cuda.synchronize()
    rows = xq if rid is None else xq[rid]
    want = np.concatenate([O.int_gemm(rows[off[e]:off[e + 1]], w[e]) for e in range(E)]).astype(np.int32)
    assert_equal(host(oi.contiguous()), want, "grouped int32")
    _pad_untouched(oi, ldo, -5, "grouped int32")
    assert_equal(_bits(ob), _bits(packed), "grouped bf16 against packed")
    _pad_untouched(ob.view(torch.int16), ldo, np.int16(0x3F00), "grouped bf16")


def _fp8_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)  # no NaN codes


@pytest.mark.parametrize("M,K,N,w_mode,kernel", [
    (2100, 384, 2100, W.FP8_W_CHANNEL, "gemm_fp8_dma_kernel<256, 128"),
    (300, 1152, 520, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 128>"),
    (2000, 384, 3100, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 256>"),
    (130, 208, 260, W.FP8_W_CHANNEL, "gemm_fp8_kernel<128, 128, false>"),
    (130, 272, 260, W.FP8_W_BLOCK128, "gemm_fp8_kernel<128, 128, true>"),
])
def test_fp8_padded(M, K, N, w_mode, kernel):
    assert W.scaled_mm_fp8_kernel_name(M, N, K, w_mode).startswith(kernel)
    rng = synth.rng_for(988, M, K, N, w_mode)
    xq, wq = _fp8_codes(rng, (M, K)), _fp8_codes(rng, (N, K))
    if w_mode == W.FP8_W_BLOCK128:
        act = W.FP8_ACT_GROUP128
        sx = rng.uniform(1e-3, 1e-1, (-(-K // 128), M)).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, (-(-N // 128), -(-K // 128))).astype(np.float32)
    else:
        act = W.FP8_ACT_TOKEN
        sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    ldx, ldw, ldo = K + 48, K + 16, N + 3
    note(f"padded fp8 M={M} K={K} N={N} w_mode={w_mode} ldo={ldo}")
    sxd, swd = to_dev(sx), to_dev(sw)
    for out_dtype, dt, fill in ((W.OUT_BF16, torch.bfloat16, 0.5), (W.OUT_F32, torch.float32, -2.0)):
        out = _out(M, N, ldo, dt, fill)
        W.scaled_mm_fp8(_padded(xq, ldx, 0x11), _padded(wq, ldw, 0x22), sxd, swd, act, w_mode,
                        out_dtype=out_dtype, out=out)
        packed = W.scaled_mm_fp8(to_dev(xq), to_dev(wq), sxd, swd, act, w_mode, out_dtype=out_dtype)
        torch.cuda.synchronize()
        if dt == torch.bfloat16:
            assert_equal(_bits(out), _bits(packed), "fp8 bf16 against packed")
            _pad_untouched(out.view(torch.int16), ldo, np.int16(0x3F00), "fp8 bf16")
        else:
            assert_equal(host(out.contiguous()).view(np.uint32), host(packed).view(np.uint32), "fp8 f32 against packed")
            _pad_untouched(out.view(torch.int32), ldo, np.float32(-2.0).view(np.int32), "fp8 f32")
