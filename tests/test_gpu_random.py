"""GPU parity on seeded random problems, through the C ABI: shapes, zero-point
modes, scale granularities, bias and output types drawn together, so that
combinations no hand-picked case names still meet the oracle. Every draw is
fixed by its seed (the same cases on every run).

* w8a8_scaled_mm_int8: M in [1, 700] (both the decode kernels and the MFMA
  tiles), K a multiple of 16 up to 2064, N up to 1600; int32 bit-exact, bf16
  within the stated bar.
* w8a8_quantize_act: every mode on ragged rows; codes, scales, zero points
  bit-exact.
* w8a8_grouped_scaled_mm_int8: random expert counts (empty experts
  included), sorted or gathered rows; int32 bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_equal, host, note, to_dev
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


@pytest.mark.parametrize("seed", range(24))
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


@pytest.mark.parametrize("seed", range(12))
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


@pytest.mark.parametrize("seed", range(8))
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
