"""Property pins of the oracle over generated inputs (CPU only).

The seeded rows of the other oracle tests come from a few normal
distributions; here hypothesis (derandomized: the same examples on every run)
draws arbitrary finite bf16 bit patterns -- subnormals, exponent extremes,
exact ties, constant rows -- and checks each oracle function against a brute
force written from the definitions in exact rational arithmetic or plain
Python loops:

* f64_to_bf16_bits: one round-to-nearest-even of the exact double to 8
  significant bits (`exact.nearest_bf16`), midpoints included;
* quant_dyn_sym / quant_dyn_asym: every IEEE step of the per-row rules
  (and rows built so that every quotient is an exact tie)
  ("MiniMax-M2.7 FP8 转昆仑芯 INT8", 转换关系; "[SGLang] W4A8, W8A8, W4A4: 혼합
  정밀도 양자화 스킴", 핵심 코드 분석 §3-§4), by the brute force of
  test_oracle_quant;
* int_gemm / colsum / corrected_acc: integer sums by Python loops;
* moe_topk / moe_sort: the ranking and the (expert, token) order by sorting
  Python tuples (ties broken by the lower expert index);
* e4m3fn_encode: the nearest OCP E4M3FN value of any binary32 in [-448, 448]
  by exhaustive search over the codes decoded from their bit fields here,
  ties to the even code, the sign kept.
"""

from fractions import Fraction

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle as O
from exact import bf16_to_fraction, nearest_bf16
from test_oracle_quant import brute_asym, brute_sym

SETTINGS = settings(derandomize=True, max_examples=150, deadline=None, database=None)

# finite bf16 bit patterns: sign, exponent 0..254, mantissa
finite_bf16 = st.integers(0, 0xFFFF).filter(lambda b: (b >> 7) & 0xFF != 0xFF)


def _bf16_rows(max_exp=254, min_len=1, max_len=24):
    """Rows of finite bf16 bits, exponent field at most max_exp."""
    elem = st.integers(0, 0xFFFF).filter(lambda b: (b >> 7) & 0xFF <= max_exp)
    return st.lists(elem, min_size=min_len, max_size=max_len)


@SETTINGS
@given(st.floats(allow_nan=False, allow_infinity=False, min_value=-3.3e38, max_value=3.3e38))
def test_f64_to_bf16_is_one_rounding(d):
    got = int(O.f64_to_bf16_bits(np.array([d]))[0])
    want = nearest_bf16(Fraction(d))
    if abs(want) > bf16_to_fraction(0x7F7F):  # past the largest finite bf16: infinity
        assert got & 0x7FFF == 0x7F80
    else:
        assert bf16_to_fraction(got) == want


@SETTINGS
@given(finite_bf16)
def test_f64_to_bf16_midpoints_go_to_even(bits):
    """The exact midpoint between a bf16 value and its neighbour above (in
    magnitude) rounds to the one with the even significand."""
    if bits & 0x7FFF == 0x7F7F:  # no finite neighbour above
        return
    mid = (bf16_to_fraction(bits) + bf16_to_fraction(bits + 1)) / 2
    d = float(mid)
    assert Fraction(d) == mid  # 9 significant bits: exact in a double
    got = int(O.f64_to_bf16_bits(np.array([d]))[0])
    assert got == (bits if bits % 2 == 0 else bits + 1)


@SETTINGS
@given(_bf16_rows())
def test_quant_dyn_sym_matches_brute_force(row):
    x = np.array([row], dtype=np.uint16)
    q, s = O.quant_dyn_sym(x)
    bq, bs = brute_sym(x[0])
    assert list(q[0]) == bq
    assert Fraction(float(s[0])) == bs


def _f32_to_bf16(v):
    bits = int(np.array([v], np.float32).view(np.uint32)[0] >> 16)
    assert bf16_to_fraction(bits) == Fraction(v)  # exact by construction
    return bits


@SETTINGS
@given(st.integers(-100, 100), st.lists(st.integers(-127, 126), min_size=1, max_size=16), st.booleans())
def test_quant_dyn_sym_ties(e, halves, neg_max):
    """Rows with absmax 127 * 2^e (so s = 2^e exactly) and values (n + 1/2) * 2^e:
    every quotient is an exact tie, which must go to the even code."""
    row = [_f32_to_bf16((-127.0 if neg_max else 127.0) * 2.0 ** e)]
    row += [_f32_to_bf16((n + 0.5) * 2.0 ** e) for n in halves]
    x = np.array([row], dtype=np.uint16)
    q, s = O.quant_dyn_sym(x)
    assert Fraction(float(s[0])) == Fraction(2) ** e
    bq, _ = brute_sym(x[0])
    assert list(q[0]) == bq
    for n, code in zip(halves, q[0, 1:]):
        assert int(code) == (n if n % 2 == 0 else n + 1)


@SETTINGS
@given(_bf16_rows(max_exp=250))  # hi - lo stays finite in binary32
def test_quant_dyn_asym_matches_brute_force(row):
    x = np.array([row], dtype=np.uint16)
    q, s, zp = O.quant_dyn_asym(x)
    bq, bs, bzp = brute_asym(x[0])
    assert list(q[0]) == bq
    assert Fraction(float(s[0])) == bs
    assert int(zp[0]) == bzp


@SETTINGS
@given(st.integers(1, 5), st.integers(1, 7), st.integers(1, 5), st.integers(0, 2 ** 31 - 1))
def test_int_gemm_colsum_and_correction_by_loops(M, K, N, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    zp = rng.integers(-128, 128, M).astype(np.int32)
    acc = O.int_gemm(q, w)
    cs = O.colsum(w)
    for t in range(M):
        for n in range(N):
            ref = sum(int(q[t, k]) * int(w[n, k]) for k in range(K))
            assert int(acc[t, n]) == ref
    for n in range(N):
        assert int(cs[n]) == sum(int(w[n, k]) for k in range(K))
    c = O.corrected_acc(acc, zp=zp, col_sum=cs)
    for t in range(M):
        for n in range(N):
            # (q - zp) . w: the asymmetric code's value times the weight
            assert int(c[t, n]) == sum((int(q[t, k]) - int(zp[t])) * int(w[n, k]) for k in range(K))


@SETTINGS
@given(st.integers(1, 6), st.integers(1, 9), st.data())
def test_moe_topk_and_sort_by_tuples(tokens, E, data):
    k = data.draw(st.integers(1, E))
    # few distinct logit values, so ties are common
    vals = data.draw(st.lists(st.sampled_from([-1.5, -0.25, 0.0, 0.5, 2.0, 3.0]), min_size=tokens * E,
                              max_size=tokens * E))
    logits = np.array(vals, np.float32).reshape(tokens, E)
    ids, wts = O.moe_topk(logits, k)
    for t in range(tokens):
        ranked = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert list(ids[t]) == ranked
        sel = [float(logits[t, e]) for e in ranked]
        ex = [np.exp(v - sel[0]) for v in sel]
        assert np.allclose(wts[t], [v / sum(ex) for v in ex], rtol=1e-15, atol=0)
    row_ids, offsets, pos = O.moe_sort(ids, E)
    pairs = sorted((int(ids[t, j]), t) for t in range(tokens) for j in range(k))
    assert [t for _, t in pairs] == list(row_ids)
    for e in range(E + 1):
        assert int(offsets[e]) == sum(1 for ex_, _ in pairs if ex_ < e)
    for t in range(tokens):
        for j in range(k):
            assert pairs[int(pos[t, j])] == (int(ids[t, j]), t)


def _e4m3_value(code):
    """Exact value of a finite E4M3FN code from its fields: sign, 4-bit
    exponent (bias 7, field 0 subnormal), 3-bit mantissa."""
    e, m = (code >> 3) & 0xF, code & 7
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if code & 0x80 else mag


_E4M3_MAGS = [(_e4m3_value(c), c) for c in range(127)]  # codes 0x00 .. 0x7E (0x7F is NaN)


@SETTINGS
@given(st.floats(min_value=-448.0, max_value=448.0, width=32, allow_nan=False))
def test_e4m3_encode_is_nearest_even(v):
    code = int(O.e4m3fn_encode(np.array([v], np.float32))[0])
    a = abs(Fraction(v))
    best = min(abs(a - m) for m, _ in _E4M3_MAGS)
    near = [c for m, c in _E4M3_MAGS if abs(a - m) == best]
    want = near[0] if len(near) == 1 else next(c for c in near if c % 2 == 0)
    if np.signbit(np.float32(v)):
        want |= 0x80
    assert code == want
    assert abs(_e4m3_value(code)) == abs(_e4m3_value(want))
