"""GPU parity of the weight-preparation calls: column sums, requantise to the
max per-tensor scale or expand it per channel, FP8 128x128-block -> per-row
int8 (all bit-exact)."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bf16_close, assert_equal, bf16_bits, host, note, to_dev
from int8_w8a8_quantized_amd import lib as W
from int8_w8a8_quantized_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 16), (130, 272), (517, 4096), (64, 14336), (3, 20016)])
def test_colsum(N, K):
    note(f"colsum N={N} K={K}")
    w = synth.rng_for(910, N, K).integers(-128, 128, (N, K), dtype=np.int8)
    got = W.prepare_colsum(to_dev(w))
    zin = torch.tensor([-37], dtype=torch.int32, device="cuda:0")
    got2 = W.prepare_colsum(to_dev(w), zp_in=zin)
    torch.cuda.synchronize()
    assert_equal(host(got), O.colsum(w), "colsum")
    assert_equal(host(got2), O.azp_adj_static(w, -37), "azp_adj")


@pytest.mark.parametrize("widths,K", [((4096, 1024, 1024), 4096), ((5, 15, 10), 48), ((33,), 272),
                                      ((7, 0, 9, 1), 64)])
def test_requant_max(widths, K):
    N = sum(widths)
    note(f"requant_max widths={widths} K={K}")
    rng = synth.rng_for(911, N, K, len(widths))
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s = rng.uniform(1e-3, 1e-2, len(widths)).astype(np.float32)
    wd = to_dev(w)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    smax = W.prepare_requant_max(wd, to_dev(s), widths, err_flag=flag)
    torch.cuda.synchronize()
    rw, rs = O.requant_max(w, s, widths)
    assert_equal(host(wd), rw, "requantised weight")
    assert host(smax)[0] == rs
    assert host(flag)[0] == 0


@pytest.mark.parametrize("widths", [(4096, 1024, 1024), (0, 5, 0, 3), (1,), tuple(range(16)), (300, 0)])
def test_expand_scales(widths):
    note(f"expand_scales widths={widths}")
    rng = synth.rng_for(913, sum(widths), len(widths))
    s = rng.uniform(1e-3, 1e-2, len(widths)).astype(np.float32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    got = W.prepare_expand_scales(to_dev(s), widths, err_flag=flag)
    torch.cuda.synchronize()
    assert_equal(host(got), O.expand_scales(s, widths), "per-channel scales")
    assert host(flag)[0] == 0
    bad = s.copy()
    bad[-1] = -1.0
    W.prepare_expand_scales(to_dev(bad), widths, err_flag=flag)
    torch.cuda.synchronize()
    assert host(flag)[0] & W.FLAG_BAD_SCALE


def test_expand_scales_then_gemm():
    """Static workload's fused QKV with its own per-partition scales, applied per channel."""
    d = synth.static_qkv()
    s_w = W.prepare_expand_scales(to_dev(d["part_scales"]), d["widths"])
    M = 37
    x = synth.rng_for(914, M, d["w"].shape[1]).integers(-128, 128, (M, d["w"].shape[1]), dtype=np.int8)
    sx = np.full(M, 0.0173, np.float32)
    out = W.scaled_mm_int8(to_dev(x), to_dev(d["w"]), to_dev(sx), s_w, out_dtype=W.OUT_I32)
    outb = W.scaled_mm_int8(to_dev(x), to_dev(d["w"]), to_dev(sx), s_w)
    torch.cuda.synchronize()
    acc = O.int_gemm(x, d["w"])
    assert_equal(host(out), acc, "accumulator")
    want = O.epilogue_bf16(acc, sx, O.expand_scales(d["part_scales"], d["widths"]))
    assert_bf16_close(bf16_bits(outb), want)


def test_requant_bad_scale_flag():
    w = np.ones((8, 16), np.int8)
    for bad in (0.0, -1.0, np.nan, np.inf):
        s = np.array([0.5, bad], np.float32)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        W.prepare_requant_max(to_dev(w), to_dev(s), (4, 4), err_flag=flag)
        torch.cuda.synchronize()
        assert host(flag)[0] & W.FLAG_BAD_SCALE


def test_requant_workload_then_azp():
    """Static workload: requantise the fused QKV, then azp_adj on the result."""
    d = synth.static_qkv()
    wd = to_dev(d["w"])
    smax = W.prepare_requant_max(wd, to_dev(d["part_scales"]), d["widths"])
    adj = W.prepare_colsum(wd, zp_in=torch.tensor([int(d["zp_in"])], dtype=torch.int32, device="cuda:0"))
    torch.cuda.synchronize()
    rw, rs = O.requant_max(d["w"], d["part_scales"], d["widths"])
    assert_equal(host(wd), rw, "requantised QKV")
    assert host(smax)[0] == rs
    assert_equal(host(adj), O.azp_adj_static(rw, int(d["zp_in"])), "azp_adj")


def _fp8_check(codes, S):
    note(f"fp8_block_to_int8 shape={codes.shape}")
    q, s, flag = W.prepare_fp8_block_to_int8(to_dev(codes), to_dev(S))
    torch.cuda.synchronize()
    rq, rs, rf = O.fp8_block_to_int8(codes, S)
    assert int(host(flag)[0]) == rf
    if rf == 0:
        assert_equal(host(q), rq, "int8 weight")
        assert_equal(host(s).view(np.uint32), rs.view(np.uint32), "row scales")


@pytest.mark.parametrize("E,N,K", [(1, 3, 16), (2, 130, 272), (3, 300, 200 - 8), (1, 256, 3072),
                                   (2, 129, 1536), (1, 5, 9216), (1, 2, 20480)])
def test_fp8_convert(E, N, K):
    codes, S = synth.fp8_block_weight(synth.rng_for(912, E, N, K), E, N, K)
    S = (S * synth.rng_for(913, E, N, K).uniform(0.25, 4.0, S.shape)).astype(np.float32)
    _fp8_check(codes, S)


# More rows than the launch has lane groups: 6144 groups of 64 lanes (K = 3072)
# or 12288 of 32 (K = 1536), so every group walks several rows through its
# two-row ring (the next row's codes and scales load while one converts).
@pytest.mark.parametrize("E,N,K", [(3, 2100, 3072), (4, 3200, 1536)])
def test_fp8_convert_rows_past_the_grid(E, N, K):
    codes, S = synth.fp8_block_weight(synth.rng_for(915, E, N, K), E, N, K)
    _fp8_check(codes, S)


def test_fp8_all_codes_and_zero_rows():
    """Every one of the 254 non-NaN codes under unit and odd scales, plus
    all-zero (and negative-zero) rows."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    row = np.concatenate([codes, codes[:2]])  # 256 codes
    m = np.stack([row, np.roll(row, 7), np.zeros(256, np.uint8), np.full(256, 0x80, np.uint8)])
    _fp8_check(m, np.array([[1.0, 3.0e-3]], np.float32))
    _fp8_check(m, np.array([[0.0, 1.0]], np.float32))  # zero scale: legal, a zero block


def test_fp8_flags():
    codes, S = synth.fp8_block_weight(synth.rng_for(914), 1, 200, 160)
    codes, S = codes[0], S[0]
    for bad in (np.nan, np.inf, -0.5):
        S2 = S.copy()
        S2[1, 1] = bad
        _fp8_check(codes, S2)
    c2 = codes.copy()
    c2[150, 3] = 0x7F
    _fp8_check(c2, S)
    S3 = S.copy()
    S3[0, 0] = 3e38
    c3 = codes.copy()
    c3[0, 0] = 0x7E
    _fp8_check(c3, S3)
