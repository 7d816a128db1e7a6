"""Pins of the oracle's MoE expert block (CPU only): routing and sorting by
brute force and a hand-worked example, the SiLU product against closed forms
and torch's float64 silu, the combine against exact rational sums, and the
whole block against a float64 MoE layer computed from the dequantised
weights. Readings: the int8 MoE method of "MiniMax-M2.7 FP8 转昆仑芯 INT8"
(版本: experts w1 / w2 / w3, w1 and w3 fused) and the w8a8 int8 MoE scheme of
"[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴" (구조도)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from exact import bf16_to_fraction, nearest_bf16
from golden_io import load_golden
from int8_w8a8_quantized_amd import synth


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_golden_routing():
    (g,) = load_golden("moe_routing_worked.txt")
    E, k = g["E"], g["k"]
    logits = np.array(g["logits"], np.float32).reshape(-1, E)
    ids, w = O.moe_topk(logits, k)
    assert ids.tolist() == np.array(g["ids"]).reshape(-1, k).tolist()
    np.testing.assert_allclose(w, np.array(g["weights"]).reshape(-1, k), rtol=1e-15, atol=0)
    row_ids, off, pos = O.moe_sort(ids, E)
    assert row_ids.tolist() == g["row_ids"]
    assert off.tolist() == g["offsets"]
    assert pos.reshape(-1).tolist() == g["pos"]


@pytest.mark.parametrize("tokens,E,k", [(7, 6, 2), (20, 64, 8), (5, 9, 9), (3, 130, 1)])
def test_topk_and_sort_brute_force(tokens, E, k):
    """Python loops: the k best experts by (larger logit, lower index), and
    the pairs listed expert by expert in token order. Logits are drawn from a
    few values so that ties are common."""
    rng = np.random.default_rng(tokens * 1000 + E)
    logits = rng.integers(-3, 4, (tokens, E)).astype(np.float32) * np.float32(0.5)
    ids, w = O.moe_topk(logits, k)
    for t in range(tokens):
        want = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert ids[t].tolist() == want
    row_ids, off, pos = O.moe_sort(ids, E)
    rows, starts = [], []
    for e in range(E):
        starts.append(len(rows))
        rows += [t for t in range(tokens) if e in ids[t].tolist()]
    starts.append(len(rows))
    assert row_ids.tolist() == rows and off.tolist() == starts
    for t in range(tokens):
        for j in range(k):
            e = int(ids[t, j])
            r = int(pos[t, j])
            assert starts[e] <= r < starts[e + 1] and rows[r] == t


def test_topk_weights_identities():
    """Weights sum to one, their ratios are exp of the logit differences, one
    expert takes weight 1 and equal logits share it equally."""
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 64)).astype(np.float32)
    ids, w = O.moe_topk(logits, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    np.testing.assert_allclose(w[:, 1:] / w[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-13)
    assert np.all(np.diff(sel, axis=1) <= 0)
    _, w1 = O.moe_topk(logits, 1)
    assert np.all(w1 == 1.0)
    _, we = O.moe_topk(np.zeros((2, 10), np.float32), 4)
    np.testing.assert_allclose(we, 0.25, rtol=1e-15)


def test_silu_closed_forms():
    """silu(0) = 0 whatever the up value; silu(1) = 1 / (1 + 1/e) =
    0.7310585786300049 and silu(-1) = -0.2689414213699951 (the logistic
    function at +-1); silu(g) -> g for large g, -> 0 for very negative g;
    a zero up value gives zero. Each within the bf16 rounding of the value."""
    h = _bf16([[0.0, 1.0, -1.0, 30.0, -30.0, 1.0, 3.0, 7.0, 2.0, 5.0],
               [2.0, 0.0, 0.0, 0.0, 0.0, 0.5, 0.5, 0.5, 0.5, 0.5]])
    a = O.bf16_bits_to_f32(O.silu_mul_bf16(h, 5)).astype(np.float64)
    want = [0.0, 0.7310585786300049 * 3.0, -0.2689414213699951 * 7.0, 30.0 * 2.0, None]
    for j in range(4):
        assert abs(a[0, j] - want[j]) <= abs(want[j]) * 2.0 ** -8
    assert 0 > a[0, 4] > -1e-10
    # silu(2) * 0.5 = 2 * 0.8807970779778823 * 0.5 (the logistic function at 2)
    assert abs(a[1, 0] - 0.8807970779778823) <= 0.8807970779778823 * 2.0 ** -8
    assert np.all(a[1, 1:5] == 0.0)


def test_silu_against_torch_float64():
    """Against torch's own float64 silu: the oracle's bf16 result is the value
    rounded once, so it lies within half a bf16 step of it."""
    rng = np.random.default_rng(4)
    inter = 96
    h = _bf16(rng.standard_normal((40, 2 * inter)).astype(np.float32) * 3)
    a = O.bf16_bits_to_f32(O.silu_mul_bf16(h, inter)).astype(np.float64)
    hf = torch.from_numpy(O.bf16_bits_to_f32(h).astype(np.float64))
    ref = (torch.nn.functional.silu(hf[:, :inter]) * hf[:, inter:]).numpy()
    step = np.ldexp(1.0, np.frexp(ref)[1] - 8)  # bf16 spacing at each value
    assert np.all(np.abs(a - ref) <= step / 2 * (1 + 1e-12))
    # and swapping the halves is far off
    swapped = (torch.nn.functional.silu(hf[:, inter:]) * hf[:, :inter]).numpy()
    assert np.max(np.abs(a - swapped)) > 1.0


def test_combine_exact_rational():
    """Each output is the exact sum of weight x expert value rounded once to
    bf16 (exact rational arithmetic on tiny inputs)."""
    rng = np.random.default_rng(5)
    tokens, k, N = 6, 3, 5
    T = tokens * k
    y = _bf16(rng.standard_normal((T, N)).astype(np.float32))
    pos = rng.permutation(T).reshape(tokens, k).astype(np.int32)
    w = rng.dirichlet(np.ones(k), tokens)
    out = O.moe_combine(y, pos, w)
    for t in range(tokens):
        for n in range(N):
            ex = sum(Fraction(float(w[t, j])) * bf16_to_fraction(int(y[pos[t, j], n])) for j in range(k))
            assert bf16_to_fraction(int(out[t, n])) == nearest_bf16(ex)


def test_combine_single_expert_is_identity():
    rng = np.random.default_rng(6)
    y = _bf16(rng.standard_normal((8, 7)).astype(np.float32))
    pos = np.arange(8, dtype=np.int32)[::-1].reshape(8, 1).copy()
    out = O.moe_combine(y, pos, np.ones((8, 1)))
    assert np.array_equal(out, y[::-1])


def _float_moe(x_bits, logits, k, w13, s13, w2, s2, swap=False):
    """A float64 MoE layer from the dequantised weights and unquantised
    activations, written with torch: softmax routing over the top k, SiLU of
    the gate rows times the up rows, then the down projection."""
    x = torch.from_numpy(O.bf16_bits_to_f32(x_bits).astype(np.float64))
    W13 = torch.from_numpy(w13.astype(np.float64) * s13[..., None].astype(np.float64))
    W2 = torch.from_numpy(w2.astype(np.float64) * s2[..., None].astype(np.float64))
    lg = torch.from_numpy(logits.astype(np.float64))
    top = torch.topk(lg, k, dim=1)
    wts = torch.softmax(top.values, dim=1)
    inter = w13.shape[1] // 2
    out = torch.zeros((x.shape[0], w2.shape[1]), dtype=torch.float64)
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(top.indices[t, j])
            h = W13[e] @ x[t]
            g, u = (h[inter:], h[:inter]) if swap else (h[:inter], h[inter:])
            out[t] += wts[t, j] * (W2[e] @ (torch.nn.functional.silu(g) * u))
    return out.numpy()


def _small_moe(seed, tokens=24, E=8, k=2, H=64, inter=32):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((tokens, H)).astype(np.float32))
    logits = rng.standard_normal((tokens, E)).astype(np.float32)
    w13 = rng.integers(-127, 128, (E, 2 * inter, H), dtype=np.int8)
    s13 = rng.uniform(1e-3, 1e-2, (E, 2 * inter)).astype(np.float32)
    w2 = rng.integers(-127, 128, (E, H, inter), dtype=np.int8)
    s2 = rng.uniform(1e-3, 1e-2, (E, H)).astype(np.float32)
    return x, logits, k, w13, s13, w2, s2


def test_block_against_float_moe_layer():
    """The int8 block approximates the float64 MoE layer on the same weights
    to within the activation quantisation noise (about 1% per row here);
    swapping the gate and up halves in the float layer misses by far more."""
    args = _small_moe(7)
    r = O.moe_block(*args)
    got = O.bf16_bits_to_f32(r["out"]).astype(np.float64)
    ref = _float_moe(*args)
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert np.max(rel) < 0.03, rel
    bad = _float_moe(*args, swap=True)
    rel_bad = np.linalg.norm(got - bad, axis=1) / np.linalg.norm(bad, axis=1)
    assert np.min(rel_bad) > 0.3, rel_bad


def test_block_steps_are_consistent():
    """Intermediates of the block: every routed row appears once, the w13
    output of a sorted row is the scaled GEMM of its token, and the w2 input
    is the per-token quantisation of the activated product."""
    x, logits, k, w13, s13, w2, s2 = _small_moe(8, tokens=10, E=5, k=3, H=32, inter=16)
    r = O.moe_block(x, logits, k, w13, s13, w2, s2)
    T = 10 * k
    assert sorted(r["pos"].reshape(-1).tolist()) == list(range(T))
    off = r["offsets"]
    for t in range(10):
        for j in range(k):
            p, e = int(r["pos"][t, j]), int(r["ids"][t, j])
            assert off[e] <= p < off[e + 1] and r["row_ids"][p] == t
            want, _ = O.scaled_mm(r["xq"][t:t + 1], w13[e], r["sx"][t:t + 1], s13[e])
            assert np.array_equal(r["h"][p:p + 1], want)
    aq, sa = O.quant_dyn_sym(r["act"])
    assert np.array_equal(aq, r["aq"]) and np.array_equal(sa, r["sa"])
