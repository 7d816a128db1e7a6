"""Pins of the oracle's W8A8 FP8 functions (CPU only): the E4M3FN encoder
against torch's float8_e4m3fn cast and against its own code table
(round trips, midpoints to the even code), the activation quantiser against
the half-step bound, the argmax and zero rules and the group/token identity,
and the FP8 GEMM (per-tensor, per-channel, 128 x 128 blocks) against exact
rational brute force. The scheme is the W8A8 FP8 one of "[SGLang] W4A8, W8A8,
W4A4: 혼합 정밀도 양자화 스킴" (핵심 코드 분석 §1-§2)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from exact import bf16_to_fraction, nearest_bf16
from int8_w8a8_quantized_amd import synth

TABLE = O.e4m3fn_table()


def test_encode_against_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(200000) * 1e-2,
                        rng.standard_normal(50000) * 1e-3, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_encode(v), want)


def test_encode_round_trip_and_midpoints():
    """Every finite code's value encodes to that code; the midpoint of two
    neighbouring magnitudes goes to the even code; a hair above it goes up,
    a hair below down."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = TABLE[codes]
    got = O.e4m3fn_encode(vals)
    assert np.array_equal(got, codes)
    mags = TABLE[:127].astype(np.float64)
    for c in range(126):
        mid = np.float32((mags[c] + mags[c + 1]) / 2)  # exact: 4 significant bits
        assert float(mid) == (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.e4m3fn_encode(np.array([mid]))[0] == even
        assert O.e4m3fn_encode(np.array([np.nextafter(mid, np.float32(1e9))]))[0] == c + 1
        assert O.e4m3fn_encode(np.array([np.nextafter(mid, np.float32(-1e9))]))[0] == c
        assert O.e4m3fn_encode(np.array([-mid]))[0] == (even | 0x80)


def _x(M, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * scale).astype(np.float32))


def _half_step(t):
    """Half the E4M3 spacing at |t| (subnormal spacing 2^-9 below 2^-6)."""
    a = np.maximum(np.abs(t.astype(np.float64)), 2.0 ** -6)
    return np.ldexp(1.0, np.frexp(a)[1] - 1 - 3) / 2


def test_quant_token_rules():
    x = _x(40, 300, 1, 3.0)
    x[3] = 0
    x[4] = 0x8000  # -0.0 throughout
    q, s = O.quant_fp8(x, O.FP8_ACT_TOKEN)
    xf = O.bf16_bits_to_f32(x)
    assert s[3] == 1 and s[4] == 1 and np.all(TABLE[q[3]] == 0) and np.all(TABLE[q[4]] == 0)
    live = [r for r in range(40) if r not in (3, 4)]
    for r in live:
        j = int(np.argmax(np.abs(xf[r])))
        assert TABLE[q[r, j]] == (448.0 if xf[r, j] > 0 else -448.0)
    t = (xf / s[:, None]).astype(np.float32)
    err = np.abs(t.astype(np.float64) - TABLE[q].astype(np.float64))
    assert np.all(err <= _half_step(t) * (1 + 2.0 ** -20))
    qn, sn = O.quant_fp8(x ^ np.uint16(0x8000), O.FP8_ACT_TOKEN)  # negated input
    assert np.array_equal(sn, s) and np.array_equal(qn, q ^ np.uint8(0x80))


def test_quant_group_equals_token_on_one_group_and_per_group_scales():
    x = _x(9, 128, 2)
    qg, sg = O.quant_fp8(x, O.FP8_ACT_GROUP128)
    qt, st = O.quant_fp8(x, O.FP8_ACT_TOKEN)
    assert sg.shape == (1, 9) and np.array_equal(sg[0], st) and np.array_equal(qg, qt)
    x = _x(5, 300, 3)
    x[1, 128:256] = 0
    q, s = O.quant_fp8(x, O.FP8_ACT_GROUP128)
    xf = O.bf16_bits_to_f32(x)
    assert s.shape == (3, 5) and s[1, 1] == 1
    for g in range(3):
        blk = xf[:, 128 * g:128 * (g + 1)]
        a = np.abs(blk).max(axis=1)
        assert np.array_equal(s[g], np.where(a == 0, 1, a / np.float32(448)).astype(np.float32))
        qt, _ = O.quant_fp8(x[:, 128 * g:128 * (g + 1)], O.FP8_ACT_TOKEN)
        assert np.array_equal(q[:, 128 * g:128 * (g + 1)], qt)


def test_quant_tensor_saturates():
    x = synth.f32_to_bf16_bits(np.array([[1.0, -1.0, 1000.0, -1000.0, 0.5, 0.0]], np.float32))
    q, s = O.quant_fp8(x, O.FP8_ACT_TENSOR, s_in=np.float32(0.5))
    assert s is None
    assert TABLE[q[0]].tolist() == [2.0, -2.0, 448.0, -448.0, 1.0, 0.0]


def _exact_mm(xq, wq, sxf, swf):
    """Exact rational out[t, n] = sum over K groups of (sum_k x w) * sx(t, g) *
    sw(n, g), and the sum of the group terms' magnitudes (the scale of the
    float64 rounding errors)."""
    M, K = xq.shape
    N = wq.shape[0]
    out = np.empty((M, N), dtype=object)
    mag = np.empty((M, N), dtype=object)
    for t in range(M):
        for n in range(N):
            tot = Fraction(0)
            m = Fraction(0)
            for g0 in range(0, K, 128):
                acc = sum(Fraction(float(TABLE[xq[t, k]])) * Fraction(float(TABLE[wq[n, k]]))
                          for k in range(g0, min(g0 + 128, K)))
                term = acc * Fraction(float(sxf(t, g0 // 128))) * Fraction(float(swf(n, g0 // 128)))
                tot += term
                m += abs(term)
            out[t, n] = tot
            mag[t, n] = m
    return out, mag


def _codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)  # no NaN codes


@pytest.mark.parametrize("w_mode,act_mode", [(O.FP8_W_CHANNEL, O.FP8_ACT_TOKEN),
                                             (O.FP8_W_TENSOR, O.FP8_ACT_TENSOR),
                                             (O.FP8_W_TENSOR, O.FP8_ACT_TOKEN),
                                             (O.FP8_W_BLOCK128, O.FP8_ACT_GROUP128)])
def test_scaled_mm_fp8_exact(w_mode, act_mode):
    rng = np.random.default_rng(10 + w_mode + act_mode)
    M, K, N = 3, 272, 130
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    G, NB = -(-K // 128), -(-N // 128)
    if w_mode == O.FP8_W_BLOCK128:
        sx = rng.uniform(1e-3, 1e-1, (G, M)).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, (NB, G)).astype(np.float32)
        sxf, swf = (lambda t, g: sx[g, t]), (lambda n, g: sw[n // 128, g])
    else:
        sx = rng.uniform(1e-3, 1e-1, M if act_mode == O.FP8_ACT_TOKEN else 1).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, N if w_mode == O.FP8_W_CHANNEL else 1).astype(np.float32)
        sxf = (lambda t, g: sx[t]) if act_mode == O.FP8_ACT_TOKEN else (lambda t, g: sx[0])
        swf = (lambda n, g: sw[n]) if w_mode == O.FP8_W_CHANNEL else (lambda n, g: sw[0])
    bias = synth.bias_bits(rng, N)
    out, y = O.scaled_mm_fp8(xq, wq, sx, sw, act_mode, w_mode, bias_bits=bias)
    ex, mag = _exact_mm(xq, wq, sxf, swf)
    for t in range(M):
        for n in range(N):
            b = bf16_to_fraction(int(bias[n]))
            e = ex[t, n] + b
            # a few float64 roundings of terms of at most this size
            assert abs(Fraction(float(y[t, n])) - e) <= (mag[t, n] + abs(b)) * Fraction(1, 2 ** 49)
            assert bf16_to_fraction(int(out[t, n])) == nearest_bf16(Fraction(float(y[t, n])))


def test_block_with_unit_scales_is_the_plain_product():
    rng = np.random.default_rng(20)
    M, K, N = 4, 384, 260
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    _, yb = O.scaled_mm_fp8(xq, wq, np.ones((3, M), np.float32), np.ones((3, 3), np.float32),
                            O.FP8_ACT_GROUP128, O.FP8_W_BLOCK128)
    _, yt = O.scaled_mm_fp8(xq, wq, np.ones(1, np.float32), np.ones(1, np.float32), O.FP8_ACT_TENSOR,
                            O.FP8_W_TENSOR)
    assert np.array_equal(yb, yt)
