"""Pins of the oracle's RMS normalisation (CPU only): torch's own float64
rms_norm, closed forms, power-of-two symmetries, the residual add against
exact rational sums, and the quantisation step of the fused form. Reading:
the quantiser takes the bf16 output of the op right before the GEMM ("[SGLang]
W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴", 핵심 코드 분석 §3); the
normalisation is the textbook RMSNorm, each bf16 result rounded once."""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle as O
from exact import bf16_to_fraction, nearest_bf16
from int8_w8a8_quantized_amd import synth


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _f64(bits):
    return O.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("M,K,eps,scale", [(3, 64, 1e-6, 3.0), (7, 4096, 1e-5, 3.0), (2, 1000, 1e-2, 3.0),
                                           (4, 128, 1e-4, 0.01)])
def test_against_torch_rms_norm(M, K, eps, scale):
    """torch.nn.functional.rms_norm in float64 on the same bf16 values: the
    oracle's bf16 result is that value rounded once, so it lies within half
    a bf16 step of it; a wrong axis or a missing weight is far off. With
    rows whose mean square is about eps (the last case) a dropped eps is off
    by about 40%."""
    rng = np.random.default_rng(M * 100 + K)
    x = _bf16(rng.standard_normal((M, K)).astype(np.float32) * np.float32(scale))
    g = _bf16(rng.uniform(0.5, 1.5, K).astype(np.float32))
    _, y = O.rmsnorm_bf16(x, g, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_f64(x)), (K,), torch.from_numpy(_f64(g)),
                                       float(np.float32(eps))).numpy()
    step = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    assert np.all(np.abs(_f64(y) - ref) <= step / 2 * (1 + 1e-9))
    no_weight = torch.nn.functional.rms_norm(torch.from_numpy(_f64(x)), (K,), None,
                                             float(np.float32(eps))).numpy()
    assert np.max(np.abs(_f64(y) - no_weight)) > 0.1


def test_closed_forms():
    """[3, 4]: mean square 12.5, y = (3, 4) / sqrt(12.5 + eps); a constant
    row c: y = c / sqrt(c^2 + eps) (about +-1); gamma scales each column."""
    eps = 1e-6
    eps32 = float(np.float32(eps))
    x = _bf16([[3.0, 4.0], [-2.0, -2.0]])
    g = _bf16([1.0, 0.5])
    _, y = O.rmsnorm_bf16(x, g, eps)
    r = math.sqrt(12.5 + eps32)
    want = [[3.0 / r, 0.5 * 4.0 / r], [-2.0 / math.sqrt(4.0 + eps32), -0.5 * 2.0 / math.sqrt(4.0 + eps32)]]
    assert np.array_equal(y, O.f64_to_bf16_bits(np.array(want)))
    assert _f64(y)[0, 0] == pytest.approx(0.8485, abs=4e-3)


def test_power_of_two_symmetries():
    """With eps far below the rows' mean square, scaling a row by 2^k leaves
    y unchanged, and scaling gamma by 2^k scales y by 2^k exactly (both
    roundings see the same significands)."""
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((5, 96)).astype(np.float32))
    g = _bf16(rng.uniform(0.5, 2.0, 96).astype(np.float32))
    eps = 1e-30
    _, y = O.rmsnorm_bf16(x, g, eps)
    for k in (-6, 3, 20):
        _, yk = O.rmsnorm_bf16(_bf16(_f64(x) * 2.0 ** k), g, eps)
        assert np.array_equal(yk, y)
        _, yg = O.rmsnorm_bf16(x, _bf16(_f64(g) * 2.0 ** k), eps)
        assert np.array_equal(_f64(yg), _f64(y) * 2.0 ** k)


def test_residual_add_exact():
    """h = x + residual rounded once to bf16 (exact rational sums), and the
    normalisation then runs on h."""
    rng = np.random.default_rng(12)
    x = _bf16(rng.standard_normal((4, 24)).astype(np.float32) * np.float32(4))
    r = _bf16(rng.standard_normal((4, 24)).astype(np.float32) * np.float32(0.01))
    r[0, :4] = _bf16([1e-30, -3.0, 0.0, 2.0 ** -12])
    g = _bf16(np.ones(24, np.float32))
    h, y = O.rmsnorm_bf16(x, g, 1e-6, residual_bits=r)
    for i in range(4):
        for j in range(24):
            ex = bf16_to_fraction(int(x[i, j])) + bf16_to_fraction(int(r[i, j]))
            assert bf16_to_fraction(int(h[i, j])) == nearest_bf16(ex)
    _, y2 = O.rmsnorm_bf16(h, g, 1e-6)
    assert np.array_equal(y, y2)
    # without the residual the input passes through as h
    h0, _ = O.rmsnorm_bf16(x, g, 1e-6)
    assert np.array_equal(h0, x)


def test_zero_row_and_eps():
    """An all-zero row normalises to zeros (its mean square is 0, eps keeps
    the quotient finite) and quantises with the all-zero-row rule."""
    x = _bf16(np.zeros((2, 16), np.float32))
    x[1, 3] = _bf16([1.0])[0]
    g = _bf16(np.ones(16, np.float32))
    _, y, q, s = O.rmsnorm_quant(x, g, 1e-6)
    assert np.all(y[0] == 0) and np.all(q[0] == 0) and s[0] == 1.0
    # the lone 1.0: mean square 1/16, y = 1 / sqrt(1/16 + eps) ~ 4, code 127
    assert _f64(y)[1, 3] == pytest.approx(4.0, rel=2 ** -8)
    assert q[1, 3] == 127 and np.count_nonzero(q[1]) == 1


def test_quant_step_is_the_quantiser():
    """The fused form's codes and scales are the per-token symmetric
    quantiser applied to its own bf16 output, which reaches 127 in magnitude
    on every nonzero row."""
    rng = np.random.default_rng(13)
    x = _bf16(rng.standard_normal((6, 256)).astype(np.float32))
    g = _bf16(rng.uniform(0.5, 1.5, 256).astype(np.float32))
    h, y, q, s = O.rmsnorm_quant(x, g, 1e-6)
    q2, s2 = O.quant_dyn_sym(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    # the scale is the row's absmax / 127 in binary32
    assert np.array_equal(s, (np.max(np.abs(O.bf16_bits_to_f32(y)), axis=1) / np.float32(127)).astype(np.float32))
    assert Fraction(float(s[0])) == Fraction(float(np.float32(np.max(np.abs(O.bf16_bits_to_f32(y[0]))) / np.float32(127))))
