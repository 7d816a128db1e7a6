"""GPU parity of the W8A8 FP8 calls against the oracle, through the C ABI.

* w8a8_quantize_act_fp8: E4M3 codes and scales bit-exact (per token, per
  tensor, per token in groups of 128).
* w8a8_scaled_mm_fp8: every kernel variant (the ring kernel's four tiles, the
  block-scaled ring kernel with 128- and 256-row tiles, the register-staged
  kernel with and without 128 x 128 block scales), against the exact sums.
  The FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) does not sum an
  instruction's 64 products exactly in binary32: it aligns them to the
  largest and truncates (measured with power-of-two operands, a product 2^14
  or more below the largest is dropped, toward zero); the accumulator input
  is added in binary32. Measured on random full-range E4M3 codes its loss is
  at most 4.8e-5 of sum_b max_b, max_b the largest possible product of 64-deep
  k block b (row max x column max); on integer-valued codes the sums are
  exact. The bars:
  - integer-valued codes in [-15, 15] (every product an integer of at most
    225, every sum exact): the binary32 output (W8A8_OUT_F32) within
    (K/64 + 4) * 2^-23 * S + 2^-21 |exact|, S the sum of the scaled
    products' magnitudes (the scale steps' roundings only);
  - full-range codes: within that plus 2^-12 * sum_b max_b (scaled), five
    times the largest loss measured; and the bf16 output within the stated
    1e-2 relative bar wherever the sum does not cancel (|exact| >= S / 16),
    within the same absolute bound plus one bf16 step elsewhere.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_equal, bf16_bits, bf16_f64, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu

assert np.array_equal(O.e4m3fn_table()[np.array([0x00, 0x38, 0x57], np.uint8)], [0.0, 1.0, 15.0])

MODES = [W.FP8_ACT_TOKEN, W.FP8_ACT_GROUP128]


def _x(M, K, seed, mean=0.0, outliers=0):
    return synth.activations(synth.rng_for(950, M, K, seed), M, K, mean, outliers, 40.0)


def _check_quant(x_bits, mode, s_in=None):
    M, K = x_bits.shape
    note(f"quantize_act_fp8 mode={mode} M={M} K={K}")
    sin = None if s_in is None else torch.tensor([s_in], dtype=torch.float32, device="cuda:0")
    q, s = W.quantize_act_fp8(to_dev(x_bits), mode, s_in=sin)
    torch.cuda.synchronize()
    rq, rs = O.quant_fp8(x_bits, mode, s_in=None if s_in is None else np.float32(s_in))
    assert_equal(host(q), rq, "E4M3 codes")
    if rs is not None:
        assert_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (16, 256), (5, 512), (7, 528), (2, 4096), (9, 8208),
                                 (1027, 1536), (2048, 4096), (300, 20480), (4, 65536)])
def test_quant_fp8_shapes(mode, M, K):
    _check_quant(_x(M, K, 1, 0.1, min(3, K)), mode)


def test_quant_fp8_edge_rows():
    """Zero and negative-zero rows, a row with one value, subnormal-range
    quotients, exact E4M3 midpoints under a unit scale, huge values."""
    K = 256
    rows = np.zeros((8, K), np.uint16)
    rows[1, :] = 0x8000
    rows[2, 17] = synth.f32_to_bf16_bits(np.array([-3.5], np.float32))[0]
    mags = O.e4m3fn_table()[:127].astype(np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    rows[3, :126] = synth.f32_to_bf16_bits(mids)
    rows[3, 126] = synth.f32_to_bf16_bits(np.array([448.0], np.float32))[0]
    rows[4] = rows[3] ^ np.uint16(0x8000)
    rows[5] = synth.f32_to_bf16_bits(np.float32(2.0 ** -12) * np.random.default_rng(0).standard_normal(K).astype(np.float32))
    rows[6] = synth.f32_to_bf16_bits(np.float32(1e30) * np.random.default_rng(1).standard_normal(K).astype(np.float32))
    rows[7, :] = np.arange(K, dtype=np.uint16) + 1  # bf16 subnormals
    for mode in MODES:
        _check_quant(rows, mode)
    _check_quant(rows[:5], W.FP8_ACT_TENSOR, s_in=1.0)  # midpoints exactly, ties to even


@pytest.mark.parametrize("s_in", [0.0213, 1e-3, 3.0])
def test_quant_fp8_tensor_saturates(s_in):
    _check_quant(_x(33, 1024, 2, 1.0, 20), W.FP8_ACT_TENSOR, s_in=s_in)


# E4M3 codes of the integers 0 .. 15
INT_CODES = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53, 0x54, 0x55, 0x56, 0x57],
                     np.uint8)


def _codes(rng, shape, narrow=False):
    """Random E4M3 codes (no NaN codes); narrow: integer values in [-15, 15]."""
    if narrow:
        return (INT_CODES[rng.integers(0, 16, shape)] | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


def _fp8_case(M, K, N, w_mode, seed, narrow=False):
    rng = synth.rng_for(951, M, K, N, w_mode, seed, int(narrow))
    xq, wq = _codes(rng, (M, K), narrow), _codes(rng, (N, K), narrow)
    G, NB = -(-K // 128), -(-N // 128)
    if w_mode == W.FP8_W_BLOCK128:
        act = W.FP8_ACT_GROUP128
        sx = rng.uniform(1e-3, 1e-1, (G, M)).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, (NB, G)).astype(np.float32)
    else:
        act = W.FP8_ACT_TOKEN if seed % 2 == 0 else W.FP8_ACT_TENSOR
        sx = rng.uniform(1e-3, 1e-1, M if act == W.FP8_ACT_TOKEN else 1).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, N if w_mode == W.FP8_W_CHANNEL else 1).astype(np.float32)
    return dict(xq=xq, wq=wq, sx=sx, sw=sw, act=act, w_mode=w_mode, bias=synth.bias_bits(rng, N),
                narrow=narrow)


def _scaled_sums(d, X, Wt):
    """sum over k of X[t,k] * Wt[n,k] with the scales applied (blockwise for
    the 128 x 128 path), float64; X, Wt non-negative here."""
    sx, sw = np.abs(d["sx"].astype(np.float64)), np.abs(d["sw"].astype(np.float64))
    M, K = X.shape
    N = Wt.shape[0]
    if d["w_mode"] == W.FP8_W_BLOCK128:
        out = np.zeros((M, N))
        for g in range(-(-K // 128)):
            out += (X[:, 128 * g:128 * g + 128] @ Wt[:, 128 * g:128 * g + 128].T) * sx[g][:, None] \
                * sw[np.arange(N) // 128, g][None, :]
        return out
    s_x = sx[:, None] if d["act"] == W.FP8_ACT_TOKEN else sx[0]
    s_w = sw[None, :] if d["w_mode"] == W.FP8_W_CHANNEL else sw[0]
    return (X @ Wt.T) * s_x * s_w


def _magnitude(d):
    """Sum over k of |scaled product|, per output (float64)."""
    tab = np.abs(O.e4m3fn_table().astype(np.float64))
    return _scaled_sums(d, tab[d["xq"]], tab[d["wq"]])


def _dropped_bound(d):
    """2^-12 times the sum over the 64-deep k blocks of the block's largest
    possible product (row max x column max), scaled: five times the most the
    MFMA's narrow internal sum was measured to lose."""
    tab = np.abs(O.e4m3fn_table().astype(np.float64))
    X, Wt = tab[d["xq"]], tab[d["wq"]]
    M, K = X.shape
    nb = -(-K // 64)
    mx = np.zeros((M, K))
    mw = np.zeros((Wt.shape[0], K))
    for b in range(nb):  # spread each block's max over the block's first column
        mx[:, 64 * b] = X[:, 64 * b:64 * b + 64].max(axis=1)
        mw[:, 64 * b] = Wt[:, 64 * b:64 * b + 64].max(axis=1)
    return 2.0 ** -12 * _scaled_sums(d, mx, mw)


def _run_fp8(d, rows=None):
    M, K = d["xq"].shape
    N = d["wq"].shape[0]
    note(f"scaled_mm_fp8 M={M} K={K} N={N} w_mode={d['w_mode']} act={d['act']} "
         f"kernel={W.scaled_mm_fp8_kernel_name(M, N, K, d['w_mode'])}")
    args = (to_dev(d["xq"]), to_dev(d["wq"]), to_dev(d["sx"]), to_dev(d["sw"]), d["act"], d["w_mode"])
    b = to_dev(d["bias"])
    y32 = W.scaled_mm_fp8(*args, bias=b, out_dtype=W.OUT_F32)
    ybf = W.scaled_mm_fp8(*args, bias=b)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(M)
    sel = dict(d)
    sel["xq"] = d["xq"][rows]
    if d["w_mode"] == W.FP8_W_BLOCK128:
        sel["sx"] = d["sx"][:, rows]
    elif d["act"] == W.FP8_ACT_TOKEN:
        sel["sx"] = d["sx"][rows]
    want_bf, want = O.scaled_mm_fp8(sel["xq"], d["wq"], sel["sx"], d["sw"], d["act"], d["w_mode"],
                                    bias_bits=d["bias"])
    mag = _magnitude(sel)
    rt = torch.from_numpy(np.asarray(rows, np.int64)).to("cuda:0")
    g32 = host(y32[rt]).astype(np.float64)
    tol = (K / 64 + 4) * 2.0 ** -23 * mag + 2.0 ** -21 * np.abs(want)
    if not d["narrow"]:
        tol = tol + _dropped_bound(sel)
    bad = np.abs(g32 - want) > tol
    assert not bad.any(), f"{int(bad.sum())} binary32 outputs outside the bound"
    gbf = bf16_f64(bf16_bits(ybf[rt]))
    obf = bf16_f64(want_bf)
    live = np.abs(want) >= mag / 16
    # elsewhere: the binary32 bound plus one bf16 step (the two roundings to
    # bf16 can land on neighbouring values, 2^-7 apart relative at most)
    step = 2.0 ** -7 * np.maximum(np.abs(obf), np.abs(gbf))
    bad = np.where(live, np.abs(gbf - obf) > 1e-2 * np.abs(obf), np.abs(gbf - obf) > tol + step)
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs outside the bar"


# (M, K, N, w_mode, kernel): each kernel the dispatch picks, ragged M and N
FP8_CASES = [
    (2300, 640, 6100, W.FP8_W_CHANNEL, "gemm_fp8_dma_kernel<256, 256, 5>"),
    (1800, 256, 5900, W.FP8_W_TENSOR, "gemm_fp8_dma_kernel<256, 192, 5>"),
    (2100, 384, 2100, W.FP8_W_CHANNEL, "gemm_fp8_dma_kernel<256, 128, 6>"),
    (300, 1152, 520, W.FP8_W_TENSOR, "gemm_fp8_dma_kernel<128, 128, 10>"),
    (37, 128, 100, W.FP8_W_CHANNEL, "gemm_fp8_dma_kernel<128, 128, 10>"),
    (130, 208, 260, W.FP8_W_CHANNEL, "gemm_fp8_kernel<128, 128, false>"),
    (5, 16, 3, W.FP8_W_TENSOR, "gemm_fp8_kernel<128, 128, false>"),
    (300, 1152, 520, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 128>"),
    (1, 128, 128, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 128>"),
    (129, 256, 129, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 128>"),
    (257, 4096, 384, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 128>"),
    (2000, 384, 3100, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 256>"),
    (1800, 256, 3968, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 256>"),
    (300, 128, 16384, W.FP8_W_BLOCK128, "gemm_fp8_block_dma_kernel<2, 256>"),
    (130, 272, 260, W.FP8_W_BLOCK128, "gemm_fp8_kernel<128, 128, true>"),
    (7, 400, 130, W.FP8_W_BLOCK128, "gemm_fp8_kernel<128, 128, true>"),
]


@pytest.mark.parametrize("M,K,N,w_mode,kernel", FP8_CASES)
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("narrow", [True, False])
def test_scaled_mm_fp8(M, K, N, w_mode, kernel, seed, narrow):
    assert W.scaled_mm_fp8_kernel_name(M, N, K, w_mode) == kernel
    _run_fp8(_fp8_case(M, K, N, w_mode, seed, narrow))


@pytest.mark.parametrize("M,K,N", [(2048, 4096, 4096), (8192, 14336, 4096)])
@pytest.mark.parametrize("w_mode", [W.FP8_W_CHANNEL, W.FP8_W_BLOCK128])
def test_scaled_mm_fp8_prefill_sizes(M, K, N, w_mode):
    """Prefill-sized products (the shapes the benchmark times), sampled rows."""
    d = _fp8_case(M, K, N, w_mode, 0)
    rng = np.random.default_rng(5)
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, M - 1} | set(rng.choice(M, 9, replace=False).tolist())))
    _run_fp8(d, rows)


def test_quant_then_gemm_chain():
    """Quantised activations straight into the GEMM, both scale layouts: the
    device codes and scales equal the oracle's, so the chain is checked too."""
    M, K, N = 96, 1024, 256
    x = _x(M, K, 3, 0.2, 5)
    rng = synth.rng_for(952)
    wq = _codes(rng, (N, K))
    for w_mode, act in ((W.FP8_W_CHANNEL, W.FP8_ACT_TOKEN), (W.FP8_W_BLOCK128, W.FP8_ACT_GROUP128)):
        q, s = W.quantize_act_fp8(to_dev(x), act)
        sw = rng.uniform(1e-4, 1e-2, N if w_mode == W.FP8_W_CHANNEL else (2, K // 128)).astype(np.float32)
        note(f"fp8 chain w_mode={w_mode}")
        out = W.scaled_mm_fp8(q, to_dev(wq), s, to_dev(sw), act, w_mode, out_dtype=W.OUT_F32)
        torch.cuda.synchronize()
        rq, rs = O.quant_fp8(x, act)
        assert_equal(host(q), rq, "codes")
        _, want = O.scaled_mm_fp8(rq, wq, rs, sw, act, w_mode)
        d = dict(xq=rq, wq=wq, sx=rs, sw=sw, act=act, w_mode=w_mode)
        tol = (K / 64 + 4) * 2.0 ** -23 * _magnitude(d) + 2.0 ** -21 * np.abs(want) + _dropped_bound(d)
        assert np.all(np.abs(host(out).astype(np.float64) - want) <= tol)


def test_mode_pairs_not_defined():
    d = _fp8_case(4, 128, 8, W.FP8_W_CHANNEL, 0)
    with pytest.raises(NotImplementedError):
        W.scaled_mm_fp8(to_dev(d["xq"]), to_dev(d["wq"]), to_dev(d["sx"]), to_dev(d["sw"]), W.FP8_ACT_GROUP128,
                        W.FP8_W_CHANNEL)
    with pytest.raises(NotImplementedError):
        W.scaled_mm_fp8(to_dev(d["xq"]), to_dev(d["wq"]), to_dev(d["sx"]), to_dev(d["sw"]), W.FP8_ACT_TOKEN,
                        W.FP8_W_BLOCK128)
