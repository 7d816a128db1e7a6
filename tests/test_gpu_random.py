"""GPU parity on seeded random problems, through the C ABI: shapes, zero-point
modes, scale granularities, bias and output types drawn together, so that
combinations no hand-picked case names still meet the oracle. Every draw is
fixed by its seed (the same cases on every run).

* w8a8_scaled_mm_int8 (48 problems): M in [1, 700] (both the decode kernels and the MFMA
  tiles), K a multiple of 16 up to 2064, N up to 1600; int32 bit-exact, bf16
  within the stated bar; and 36 more with K a multiple of 128 (or 64) on
  the main decode kernels and MFMA tiles, up to 2599 x 8192 x 6499.
* w8a8_quantize_act: every mode on ragged rows; codes, scales, zero points
  bit-exact.
* w8a8_grouped_scaled_mm_int8: random expert counts (empty experts
  included), sorted or gathered rows; int32 bit-exact.
* w8a8_scaled_mm_fp8 (every weight-scale layout, ring and register-staged
  kernels) to the bounds of test_gpu_fp8;
* w8a8_quantize_act_fp8 (every mode), w8a8_linear_dyn_sym (fused and
  two-launch shapes) and w8a8_rmsnorm_quant (with and without a residual),
  each to the bar of its own test file.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, bf16_f64, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth
from test_gpu_gemm import _run

pytestmark = pytest.mark.gpu


def _gemm_draw(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([rng.integers(1, 129), rng.integers(129, 701)]))
    K = int(rng.integers(1, 130)) * 16
    N = int(rng.integers(1, 1601))
    return M, K, N, rng


@pytest.mark.parametrize("seed", range(48))
def test_scaled_mm_random(seed):
    M, K, N, rng = _gemm_draw(seed)
    azp = int(rng.integers(0, 3))
    per_token, per_channel, bias = bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    d = dict(
        xq=rng.integers(-128, 128, (M, K), dtype=np.int8),
        w=rng.integers(-128, 128, (N, K), dtype=np.int8),
        sx=rng.uniform(1e-3, 5e-2, M).astype(np.float32),
        sw=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
        zp=rng.integers(-128, 128, M).astype(np.int32),
        bias=synth.bias_bits(rng, N),
        zin=int(rng.integers(-128, 128)),
    )
    note(f"random scaled_mm seed={seed} M={M} K={K} N={N} azp={azp} kernel={W.scaled_mm_kernel_name(M, N, K)}")
    _run(d, azp, per_token=per_token, per_channel=per_channel, out_dtype=W.OUT_I32)
    _run(d, azp, per_token=per_token, per_channel=per_channel, bias=bias)


def _gemm_draw_main(seed):
    """K a multiple of 128 (of 64 for some large problems), so the draws land
    on the main kernels: decode (M <= 128, N up to 9000, K up to 8192),
    middle (M 129-999) and large (M 1000-2599, N 2000-6499) problems."""
    rng = np.random.default_rng(1500 + seed)
    cls = seed % 3
    if cls == 0:
        M, K, N = int(rng.integers(1, 129)), int(rng.integers(1, 65)) * 128, int(rng.integers(1, 9000))
    elif cls == 1:
        M, K, N = int(rng.integers(129, 1000)), int(rng.integers(1, 33)) * 128, int(rng.integers(1, 3000))
    else:
        M, K, N = (int(rng.integers(1000, 2600)), int(rng.integers(1, 9)) * (128 if rng.random() < 0.7 else 64),
                   int(rng.integers(2000, 6500)))
    return M, K, N, rng


@pytest.mark.parametrize("seed", range(36))
def test_scaled_mm_random_main_kernels(seed):
    M, K, N, rng = _gemm_draw_main(seed)
    azp = int(rng.integers(0, 3))
    per_token, per_channel, bias = bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    d = dict(
        xq=rng.integers(-128, 128, (M, K), dtype=np.int8),
        w=rng.integers(-128, 128, (N, K), dtype=np.int8),
        sx=rng.uniform(1e-3, 5e-2, M).astype(np.float32),
        sw=rng.uniform(1e-3, 1e-2, N).astype(np.float32),
        zp=rng.integers(-128, 128, M).astype(np.int32),
        bias=synth.bias_bits(rng, N),
        zin=int(rng.integers(-128, 128)),
    )
    note(f"random scaled_mm (main kernels) seed={seed} M={M} K={K} N={N} azp={azp} "
         f"kernel={W.scaled_mm_kernel_name(M, N, K)}")
    _run(d, azp, per_token=per_token, per_channel=per_channel, out_dtype=W.OUT_I32)
    _run(d, azp, per_token=per_token, per_channel=per_channel, bias=bias)


@pytest.mark.parametrize("seed", range(24))
def test_quantize_act_random(seed):
    rng = np.random.default_rng(2000 + seed)
    M = int(rng.integers(1, 600))
    K = int(rng.integers(1, 150)) * 16
    mode = int(rng.integers(0, 4))
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(rng.uniform(0.01, 30.0))
    x += np.float32(rng.uniform(-1, 1))
    xb = synth.f32_to_bf16_bits(x)
    s_in = zp_in = None
    if mode in (W.QUANT_STATIC_SYM, W.QUANT_STATIC_ASYM):
        s_in = np.float32(np.abs(x).max() / 100.0 + 1e-6)
        zp_in = int(rng.integers(-128, 128)) if mode == W.QUANT_STATIC_ASYM else 0
    note(f"random quantize_act seed={seed} M={M} K={K} mode={mode}")
    sd = None if s_in is None else torch.tensor([s_in], dtype=torch.float32, device="cuda:0")
    zd = None if zp_in is None else torch.tensor([zp_in], dtype=torch.int32, device="cuda:0")
    q, s, zp = W.quantize_act(to_dev(xb), mode, s_in=sd, zp_in=zd)
    torch.cuda.synchronize()
    rq, rs, rzp = O.quantize_act(xb, mode, s_in=s_in, zp_in=zp_in)
    assert_equal(host(q), rq, "codes")
    if rs is not None:
        assert_equal(host(s).view(np.uint32), np.asarray(rs, np.float32).view(np.uint32), "scales")
    if rzp is not None:
        assert_equal(host(zp), np.asarray(rzp, np.int32), "zero points")


@pytest.mark.parametrize("seed", range(16))
def test_grouped_random(seed):
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.integers(1, 70))
    K = int(rng.integers(1, 40)) * 16
    N = int(rng.integers(1, 700))
    counts = rng.integers(0, 400, E) * (rng.random(E) < 0.8)  # some experts empty
    T = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    gather = bool(rng.integers(0, 2))
    M_src = int(rng.integers(1, 500)) if gather else T
    xq = rng.integers(-128, 128, (max(M_src, 1), K), dtype=np.int8)[:M_src]
    rid = rng.integers(0, max(M_src, 1), T).astype(np.int32) if gather else None
    w = rng.integers(-128, 128, (E, N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 5e-2, max(M_src, 1)).astype(np.float32)[:M_src]
    sw = rng.uniform(1e-3, 1e-2, (E, N)).astype(np.float32)
    note(f"random grouped seed={seed} E={E} T={T} K={K} N={N} gather={gather}")
    out = W.grouped_scaled_mm_int8(to_dev(xq), to_dev(off), to_dev(w), to_dev(sx), to_dev(sw),
                                   row_ids=None if rid is None else to_dev(rid), T=T, out_dtype=W.OUT_I32)
    torch.cuda.synchronize()
    rows = xq if rid is None else xq[rid]
    want = np.zeros((T, N), np.int64)
    for e in range(E):
        if off[e + 1] > off[e]:
            want[off[e]:off[e + 1]] = O.int_gemm(rows[off[e]:off[e + 1]], w[e])
    assert_equal(host(out), want.astype(np.int32), "grouped int32")


@pytest.mark.parametrize("seed", range(8))
def test_quantize_act_fp8_random(seed):
    rng = np.random.default_rng(4000 + seed)
    M = int(rng.integers(1, 400))
    K = int(rng.integers(1, 100)) * 16
    mode = int(rng.integers(0, 3))
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(rng.uniform(0.01, 50.0))
    xb = synth.f32_to_bf16_bits(x)
    s_in = np.float32(np.abs(x).max() / 300.0 + 1e-6) if mode == W.FP8_ACT_TENSOR else None
    note(f"random quantize_act_fp8 seed={seed} M={M} K={K} mode={mode}")
    sd = None if s_in is None else torch.tensor([s_in], dtype=torch.float32, device="cuda:0")
    q, s = W.quantize_act_fp8(to_dev(xb), mode, s_in=sd)
    torch.cuda.synchronize()
    rq, rs = O.quant_fp8(xb, mode, s_in=s_in)
    assert_equal(host(q), rq, "E4M3 codes")
    if rs is not None:
        assert_equal(host(s).view(np.uint32), np.asarray(rs, np.float32).view(np.uint32), "scales")


@pytest.mark.parametrize("seed", range(8))
def test_linear_dyn_sym_random(seed):
    """Quantiser + GEMM in one call (one fused kernel on the smallest shapes):
    codes and scales bit-exact, the output within the bar."""
    rng = np.random.default_rng(5000 + seed)
    M = int(rng.choice([rng.integers(1, 3), rng.integers(3, 129)]))
    K = int(rng.integers(1, 80)) * 128 if rng.random() < 0.7 else int(rng.integers(1, 300)) * 16
    N = int(rng.integers(1, 5000))
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * np.float32(2.0))
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    bias = synth.bias_bits(rng, N)
    note(f"random linear_dyn_sym seed={seed} M={M} K={K} N={N} kernel={W.linear_dyn_sym_kernel_name(M, N, K)}")
    out, xq, sx = W.linear_dyn_sym(to_dev(x), to_dev(w), to_dev(sw), bias=to_dev(bias))
    torch.cuda.synchronize()
    rq, rs = O.quant_dyn_sym(x)
    assert_equal(host(xq), rq, "codes")
    assert_equal(host(sx).view(np.uint32), rs.view(np.uint32), "scales")
    want, _ = O.scaled_mm(rq, w, rs, sw, bias_bits=bias)
    assert_bf16_close(bf16_bits(out), want)


@pytest.mark.parametrize("seed", range(6))
def test_rmsnorm_quant_random(seed):
    """The residual sum bit-exact; codes and scales bit-exact against the
    quantiser applied to the device's own normalised rows, which must equal
    the oracle's wherever no value sits within 2^-40 of a bf16 midpoint."""
    rng = np.random.default_rng(6000 + seed)
    M = int(rng.integers(1, 300))
    K = int(rng.integers(1, 400)) * 16
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * np.float32(rng.uniform(0.1, 10)))
    g = synth.f32_to_bf16_bits(rng.uniform(0.2, 2.0, K).astype(np.float32))
    r = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)) if rng.random() < 0.5 else None
    eps = float(rng.choice([1e-6, 1e-5]))
    note(f"random rmsnorm_quant seed={seed} M={M} K={K} residual={r is not None}")
    rd = None if r is None else to_dev(r)
    xq, sx, y = W.rmsnorm_quant(to_dev(x), to_dev(g), eps, residual=rd, want_y=True)
    torch.cuda.synchronize()
    h_ref, y_ref = O.rmsnorm_bf16(x, g, eps, residual_bits=r)
    if r is not None:
        assert_equal(bf16_bits(rd), h_ref, "residual sum")
    y_dev = bf16_bits(y)
    diff = y_dev != y_ref
    if diff.any():  # only the midpoint ambiguity of the binary64 evaluation is allowed
        h = O.bf16_bits_to_f32(h_ref).astype(np.float64)
        gg = O.bf16_bits_to_f32(g).astype(np.float64)
        exact = (h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + float(np.float32(eps))) * gg[None, :])[diff]
        mid = (bf16_f64(y_dev[diff]) + bf16_f64(y_ref[diff])) / 2
        assert np.all(np.abs(exact - mid) <= 2.0 ** -40 * np.abs(exact)), "normalised rows differ"
    q_ref, s_ref = O.quant_dyn_sym(y_dev)
    assert_equal(host(xq), q_ref, "codes")
    assert_equal(host(sx).view(np.uint32), s_ref.view(np.uint32), "scales")


@pytest.mark.parametrize("seed", range(20))
def test_scaled_mm_fp8_random(seed):
    """The W8A8 FP8 GEMM on random shapes and scale layouts, to the bounds of
    test_gpu_fp8 (integer-valued codes: the scale steps' roundings only; full
    range: plus the measured summation loss)."""
    from test_gpu_fp8 import _fp8_case, _run_fp8
    rng = np.random.default_rng(7000 + seed)
    M = int(rng.integers(1, 600))
    K = int(rng.integers(1, 30)) * (128 if rng.random() < 0.7 else 16)
    N = int(rng.integers(1, 1200))
    w_mode = int(rng.integers(0, 3))
    _run_fp8(_fp8_case(M, K, N, w_mode, seed, narrow=bool(seed % 2)))
