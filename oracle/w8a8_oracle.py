"""Plain CPU oracle of the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module. The HIP library shares no code with it.

Written with numpy only, for clarity rather than speed. Sources, by page title:

* [vLLM]    "vLLM INT8 W8A8 量化实战：用 llm-compressor 制作 8 位权重与 8 位激活的推理模型"
* [SGLang]  "[SGLang] W4A8, W8A8, W4A4: 혼합 정밀도 양자화 스킴"
* [Kunlun]  "MiniMax-M2.7 FP8 转昆仑芯 INT8" (README of minimax-m2-kunlun-INT8)

Precision. Where a float decides an integer (a quantised code, a scale that
feeds one) the step is done in IEEE binary32 with round-to-nearest-even, the
precision the [Kunlun] conversion formulas name (``W_fp32``). Every such step
is one numpy float32 op, so each result is the correctly rounded binary32
value of that op. Integer sums are exact (int64, or float64 where every
partial sum stays below 2**53). The one floating-point *output*, the
dequantised bf16 result, is computed in float64 from the exact integer
accumulator and then rounded once to bf16 (round-to-nearest-even).

Readings of points the pages leave open:

* ``round`` is round-half-to-even (numpy ``rint``); the division by a scale is a
  true IEEE division, never a multiply by a reciprocal.
* Per-token symmetric activation quantisation applies the per-row absmax/127
  rule of [Kunlun] 转换关系 to each token row; an all-zero row gives q=0, s=1
  (the same page's all-zero-row rule).
* Asymmetric activation quantisation is the textbook affine mapping onto
  [-128, 127] with the range widened to contain 0: s=(hi-lo)/255,
  zp=-128-rne(lo/s), q=clamp(rne(x/s)+zp). The pages only say that the zero
  point exists, is stored as int8 and is used as an int32 "azp" ([vLLM] 4.2).
* The zero point is subtracted: x ~ s*(q-zp), so the integer correction is
  acc - zp*colsum(W) ([SGLang] 핵심 코드 분석 §4).
* requantize-with-max-scale dequantises each partition with its own scale and
  quantises again with the largest one ([SGLang] §7); range [-128, 127].

Pins (``tests/test_oracle_*.py``, run with ``-m "not gpu"``): exact rational
brute force of every rounding decision on small rows, the half-step error
bound, the argmax/argmin mapping, sign and power-of-two symmetries, the
all-zero-row rule, a pure-Python integer GEMM, the dequantise-then-matmul
identity, the OCP E4M3FN decoding against torch's float8_e4m3fn and hand
values, hand-computed worked examples under ``tests/golden/``, for the MoE
block: brute-force routing and sorting, closed forms and identities of the
SiLU product and the combine, and the whole block against a float64
dequantise-then-compute MoE layer; for the RMS normalisation: torch's
float64 rms_norm, closed forms, power-of-two symmetries and the residual add
against exact rational sums.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f32",
    "f64_to_bf16_bits",
    "quant_dyn_sym",
    "quant_dyn_asym",
    "quant_static",
    "quantize_act",
    "int_gemm",
    "colsum",
    "azp_adj_static",
    "corrected_acc",
    "epilogue_bf16",
    "scaled_mm",
    "requant_max",
    "expand_scales",
    "e4m3fn_table",
    "fp8_block_to_int8",
    "grouped_scaled_mm",
    "e4m3fn_encode",
    "quant_fp8",
    "scaled_mm_fp8",
    "FP8_MAX",
    "FP8_ACT_TOKEN",
    "FP8_ACT_TENSOR",
    "FP8_ACT_GROUP128",
    "FP8_W_TENSOR",
    "FP8_W_CHANNEL",
    "FP8_W_BLOCK128",
    "moe_topk",
    "moe_sort",
    "silu_mul_bf16",
    "rmsnorm_bf16",
    "rmsnorm_quant",
    "moe_combine",
    "moe_block",
    "linear_forward",
    "FLAG_NAN_CODE",
    "FLAG_BAD_SCALE",
    "FLAG_NONFINITE",
    "MODE_DYN_SYM",
    "MODE_DYN_ASYM",
    "MODE_STATIC_SYM",
    "MODE_STATIC_ASYM",
]

MODE_DYN_SYM = 0
MODE_DYN_ASYM = 1
MODE_STATIC_SYM = 2
MODE_STATIC_ASYM = 3

FLAG_NAN_CODE = 1   # an FP8 NaN code (0x7F / 0xFF) in the weight
FLAG_BAD_SCALE = 2  # a scale that is NaN, +-Inf or negative
FLAG_NONFINITE = 4  # a dequantised value that overflowed binary32

_F = np.float32


# ---------------------------------------------------------------- bf16 I/O --

def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32. Exact: bf16 is the top half of binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_bf16_bits(y) -> np.ndarray:
    """Round float64 values once to bf16 (round-to-nearest-even) and return the bits.

    bf16 has binary32's exponent range and 8 significant bits. For a finite y,
    write |y| = m * 2**e with m in [0.5, 1); the nearest bf16 is
    rint(m * 2**8) * 2**(e-8) in the normal range, and a multiple of 2**-133
    (the smallest bf16 subnormal) below 2**-126. Beyond the largest finite bf16
    the rounding overflows to infinity.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.float64)
    fin = np.isfinite(y)
    m, e = np.frexp(np.where(fin, y, 0.0))
    quantum_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(np.where(fin, y, 0.0), -quantum_exp))  # exact scaling, RNE
    out[...] = np.ldexp(r, quantum_exp)
    out[~fin] = y[~fin]
    max_bf16 = float(np.ldexp(255.0, 127 - 7))  # (2 - 2**-7) * 2**127
    over = fin & (np.abs(out) > max_bf16)
    out[over] = np.copysign(np.inf, y[over])
    # binary32 holds every bf16 value exactly, so the bits are its top half.
    f32 = out.astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------- activation quantisation --

def quant_dyn_sym(x_bits):
    """Dynamic per-token symmetric int8 quantisation of bf16 activations [M, K].

    Follows the per-row absmax rule of [Kunlun] 转换关系, applied to token rows,
    as used by the per-token quantiser of [SGLang] 핵심 코드 분석 §3:
        s_t = max_k |x_tk| / 127,   q = clamp(round(x / s_t), -127, 127),
    with an all-zero row giving q = 0 and s = 1 ([Kunlun] 转换关系).
    Returns (q int8 [M,K], s float32 [M]).
    """
    x = bf16_bits_to_f32(x_bits)
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], _F)
    s = np.where(a == 0, _F(1), a / _F(127)).astype(_F)
    r = np.rint(x / s[:, None])
    q = np.clip(r, -127, 127).astype(np.int8)
    return q, s


def quant_dyn_asym(x_bits):
    """Dynamic per-token asymmetric int8 quantisation with a zero point.

    The pages state that asymmetric input quantisation is supported and that the
    zero point is an int8 used as int32 ([vLLM] 4.2; [SGLang] §3-§4); the
    mapping itself is the affine one over [-128, 127] with [lo, hi] widened to
    contain zero:
        lo = min(0, min x), hi = max(0, max x), s = (hi - lo) / 255,
        zp = clamp(-128 - round(lo / s), -128, 127),
        q  = clamp(round(x / s) + zp, -128, 127).
    Row all zero (hi == lo): s = 1, zp = 0, q = 0.
    Returns (q int8 [M,K], s float32 [M], zp int32 [M]).
    """
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    if K:
        lo = np.minimum(_F(0), np.min(x, axis=1)).astype(_F)
        hi = np.maximum(_F(0), np.max(x, axis=1)).astype(_F)
    else:
        lo = np.zeros(M, _F)
        hi = np.zeros(M, _F)
    zero_row = hi == lo
    rng = (hi - lo).astype(_F)
    s = np.where(zero_row, _F(1), rng / _F(255)).astype(_F)
    zp = -128 - np.rint(lo / s).astype(np.int64)
    zp = np.clip(zp, -128, 127)
    zp = np.where(zero_row, 0, zp)
    r = np.rint(x / s[:, None]).astype(np.float64)
    q = np.clip(r + zp[:, None], -128, 127).astype(np.int8)
    return q, s, zp.astype(np.int32)


def quant_static(x_bits, s_in, zp_in=0, symmetric=True):
    """Static per-tensor quantisation with a calibrated scale (and zero point).

    [vLLM] 4.1 (static tensor-wise input scale) and 4.2 (input_scale /
    input_zero_point registered only for static input):
        q = clamp(round(x / s_in) + zp_in, qmin, qmax),
    [-127, 127] with zp_in = 0 when symmetric, [-128, 127] otherwise.
    The sum is exact integer arithmetic on the rounded quotient.
    """
    x = bf16_bits_to_f32(x_bits)
    s = _F(s_in)
    r = np.rint(x / s).astype(np.float64)
    if symmetric:
        return np.clip(r, -127, 127).astype(np.int8)
    return np.clip(r + int(zp_in), -128, 127).astype(np.int8)


def quantize_act(x_bits, mode, s_in=None, zp_in=None):
    """Dispatch on the four activation modes. Returns (q, s or None, zp or None)."""
    if mode == MODE_DYN_SYM:
        q, s = quant_dyn_sym(x_bits)
        return q, s, None
    if mode == MODE_DYN_ASYM:
        return quant_dyn_asym(x_bits)
    if mode == MODE_STATIC_SYM:
        return quant_static(x_bits, s_in, 0, True), None, None
    if mode == MODE_STATIC_ASYM:
        return quant_static(x_bits, s_in, zp_in, False), None, None
    raise ValueError(f"unknown mode {mode}")


# -------------------------------------------------------------- the GEMM --

def int_gemm(q, w):
    """acc[t, n] = sum_k q[t,k] * w[n,k], exact, as int64.

    [SGLang] §3 (int8 x int8 matrix product) with the [vLLM] 4.2 weight layout
    [out_features, in_features]. Computed as a float64 matrix product: every
    product is below 2**14 in magnitude and every partial sum below
    K * 2**14 < 2**53 for K < 2**39, so any summation order is exact.
    """
    q = np.asarray(q, dtype=np.int8)
    w = np.asarray(w, dtype=np.int8)
    assert q.shape[1] == w.shape[1]
    acc = q.astype(np.float64) @ w.astype(np.float64).T
    return acc.astype(np.int64)


def colsum(w):
    """colsum[n] = sum_k W[n, k] as int32 ([SGLang] §4: the weight sum over the
    input dimension, which is dim 0 of the transposed [K, N] weight)."""
    return np.asarray(w, dtype=np.int8).astype(np.int64).sum(axis=1).astype(np.int32)


def azp_adj_static(w, zp_in):
    """Static asymmetric input: azp_adj = input_zero_point * colsum ([SGLang] §4)."""
    return (np.int64(zp_in) * colsum(w).astype(np.int64)).astype(np.int32)


def corrected_acc(acc, zp=None, col_sum=None, azp_adj=None):
    """Integer zero-point correction c = acc - zp_t*colsum_n (dynamic asym), or
    c = acc - azp_adj_n (static asym), or c = acc ([SGLang] §4)."""
    c = np.asarray(acc, dtype=np.int64)
    if zp is not None:
        c = c - np.asarray(zp, np.int64)[:, None] * np.asarray(col_sum, np.int64)[None, :]
    elif azp_adj is not None:
        c = c - np.asarray(azp_adj, np.int64)[None, :]
    return c


def epilogue_bf16(c, s_x, s_w, bias_bits=None):
    """out = bf16(c * s_x[t] * s_w[n] + bias[n]).

    [SGLang] §3: the integer product is scaled by the token scale and the
    weight scale, the bias is added and the result is returned in the input's
    dtype (bf16). s_x / s_w may be scalars (per-tensor) or vectors. The value
    is formed in float64 and rounded once to bf16.
    """
    c = np.asarray(c, dtype=np.float64)
    sx = np.asarray(s_x, dtype=np.float32).astype(np.float64)
    sw = np.asarray(s_w, dtype=np.float32).astype(np.float64)
    sx = sx.reshape(-1, 1) if sx.ndim else sx
    sw = sw.reshape(1, -1) if sw.ndim else sw
    y = c * sx * sw
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return f64_to_bf16_bits(y)


def scaled_mm(q, w, s_x, s_w, zp=None, azp_adj=None, bias_bits=None):
    """The scaled int8 GEMM with its fused epilogue ([SGLang] §3-§4).

    Returns (out bf16 bits [M,N], c int64 [M,N]) where c is the corrected
    integer accumulator.
    """
    acc = int_gemm(q, w)
    cs = colsum(w) if zp is not None else None
    c = corrected_acc(acc, zp=zp, col_sum=cs, azp_adj=azp_adj)
    return epilogue_bf16(c, s_x, s_w, bias_bits), c


def linear_forward(x_bits, w, s_w, mode, s_in=None, zp_in=None, bias_bits=None):
    """quantize_act then scaled_mm, the forward of the W8A8 linear layer
    ([SGLang] §3 apply_weights). Returns the bf16 output bits."""
    q, s, zp = quantize_act(x_bits, mode, s_in, zp_in)
    if mode == MODE_DYN_SYM:
        out, _ = scaled_mm(q, w, s, s_w, bias_bits=bias_bits)
    elif mode == MODE_DYN_ASYM:
        out, _ = scaled_mm(q, w, s, s_w, zp=zp, bias_bits=bias_bits)
    elif mode == MODE_STATIC_SYM:
        out, _ = scaled_mm(q, w, _F(s_in), s_w, bias_bits=bias_bits)
    else:
        out, _ = scaled_mm(q, w, _F(s_in), s_w,
                           azp_adj=azp_adj_static(w, zp_in), bias_bits=bias_bits)
    return out


# ------------------------------------------------------ weight preparation --

def requant_max(w, part_scales, logical_widths):
    """Requantise a fused weight with one scale per partition to the largest scale.

    [SGLang] §7 (requantize_with_max_scale): the rows of partition p
    (logical_widths gives each partition's row count) are dequantised with
    their own scale s_p and quantised again with s_max = max_p s_p:
        d = fp32(W * s_p),  W' = clamp(round(d / s_max), -128, 127).
    Returns (W' int8 [N,K], s_max float32).
    """
    w = np.asarray(w, dtype=np.int8)
    ps = np.asarray(part_scales, dtype=np.float32)
    widths = [int(v) for v in logical_widths]
    assert sum(widths) == w.shape[0] and len(widths) == ps.shape[0]
    s_max = _F(np.max(ps))
    out = np.empty_like(w)
    r0 = 0
    for p, width in enumerate(widths):
        rows = w[r0:r0 + width].astype(np.float32)
        d = rows * ps[p]
        out[r0:r0 + width] = np.clip(np.rint(d / s_max), -128, 127).astype(np.int8)
        r0 += width
    return out, s_max


def expand_scales(part_scales, logical_widths):
    """Per-output-channel scales of a fused weight from its per-partition scales.

    [SGLang] §7 tracks each partition's rows through logical_widths, and §4's
    is_channelwise selects a per-channel weight scale; giving every row of
    partition p the scale s_p keeps each partition's own dequantisation
    W * s_p exactly (no requantisation to the largest scale):
        s_w[n] = s_p  for the rows n of partition p.
    Returns float32 [N].
    """
    ps = np.asarray(part_scales, dtype=np.float32)
    widths = [int(v) for v in logical_widths]
    assert len(widths) == ps.shape[0] and all(v >= 0 for v in widths)
    return np.repeat(ps, widths).astype(np.float32)


def e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3FN code as float32 (NaN for 0x7F and 0xFF).

    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    encodes subnormals 2**-6 * m/8; exponent 15 with mantissa 7 is NaN and
    there is no infinity, so the largest finite value is 1.75 * 2**8 = 448.
    """
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t.astype(np.float32)


def fp8_block_to_int8(w8, scales, block=128):
    """FP8 128x128 block-scaled weight -> per-row symmetric int8 ([Kunlun] 转换关系).

        W32[i,j] = fp32(dec(W8[i,j]) * S[i//128, j//128])   (the stored "_inv"
                   scale multiplies; it is not inverted)
        s[i]     = fp32(max_j |W32[i,j]| / 127)
        q[i,j]   = clamp(round(W32[i,j] / s[i]), -127, 127)
    An all-zero row gives q = 0, s = 1. w8 is uint8 codes [N,K] or [E,N,K];
    scales is float32 [ceil(N/128), ceil(K/128)] (or with a leading E).
    Returns (q int8, s float32 [.., N], flags int) where flags ORs
    FLAG_NAN_CODE, FLAG_BAD_SCALE (NaN, +-Inf or negative scale, the page's
    "illegal scale" of 验证) and FLAG_NONFINITE. Outputs are unspecified when
    flags is non-zero.
    """
    w8 = np.asarray(w8, dtype=np.uint8)
    S = np.asarray(scales, dtype=np.float32)
    if w8.ndim == 3:
        qs, ss, fl = [], [], 0
        for e in range(w8.shape[0]):
            q, s, f = fp8_block_to_int8(w8[e], S[e], block)
            qs.append(q)
            ss.append(s)
            fl |= f
        N, K = w8.shape[1:]
        return (np.stack(qs) if qs else np.zeros((0, N, K), np.int8),
                np.stack(ss) if ss else np.zeros((0, N), np.float32), fl)
    N, K = w8.shape
    nb, kb = -(-N // block), -(-K // block)
    assert S.shape == (nb, kb), (S.shape, (nb, kb))
    flags = 0
    if np.any((w8 & 0x7F) == 0x7F):
        flags |= FLAG_NAN_CODE
    if np.any(~np.isfinite(S) | (S < 0)):
        flags |= FLAG_BAD_SCALE
    dec = e4m3fn_table()[w8]
    S_full = np.repeat(np.repeat(S, block, axis=0), block, axis=1)[:N, :K]
    with np.errstate(invalid="ignore", over="ignore"):
        w32 = (dec * S_full).astype(np.float32)
    if np.any(~np.isfinite(w32) & ~np.isnan(dec) & np.isfinite(S_full)):
        flags |= FLAG_NONFINITE
    with np.errstate(invalid="ignore"):
        a = np.max(np.abs(w32), axis=1) if K else np.zeros(N, np.float32)
    s = np.where(a == 0, _F(1), a / _F(127)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.rint(w32 / s[:, None])
    q = np.clip(np.nan_to_num(r), -127, 127).astype(np.int8)
    return q, s, flags


# ---------------------------------------------------------------- MoE --

def grouped_scaled_mm(xq, s_x, w, s_w, expert_offsets, row_ids=None, bias_bits=None):
    """Grouped (MoE) scaled GEMM: for each expert e, the rows [off_e, off_e+1)
    of the expert-sorted activation take the plain scaled GEMM with W[e], s_w[e]
    (and bias[e]); [SGLang] 구조도 (the w8a8_int8 MoE scheme) and [Kunlun] 版本
    (the int8 MoE method over experts w1/w2/w3).

    row_ids (optional) gathers row r of the sorted order from xq[row_ids[r]]
    and s_x[row_ids[r]]; without it xq / s_x are already in sorted order.
    Returns (out bf16 bits [T,N], c int64 [T,N]).
    """
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = w.shape[0]
    assert off.shape == (E + 1,) and off[0] == 0 and np.all(np.diff(off) >= 0)
    T, N = int(off[-1]), w.shape[1]
    out = np.zeros((T, N), dtype=np.uint16)
    cc = np.zeros((T, N), dtype=np.int64)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        rows = np.asarray(row_ids[r0:r1], np.int64) if row_ids is not None else np.arange(r0, r1)
        b = None if bias_bits is None else bias_bits[e]
        o, c = scaled_mm(xq[rows], w[e], np.asarray(s_x)[rows], s_w[e], bias_bits=b)
        out[r0:r1] = o
        cc[r0:r1] = c
    return out, cc


# ------------------------------------------------------- MoE expert block --
#
# The int8 MoE method of [Kunlun] 版本 keeps the experts' w1 / w2 / w3, which
# vLLM fuses (w1 and w3 into one w13) and runs with per-token dynamic
# symmetric int8 activations and per-output-channel symmetric int8 weights;
# [SGLang] 구조도 lists the same scheme (the w8a8_int8 MoE). The pages give
# no formula for the routing, the activation between w13 and w2 or the
# combine; the readings below are the plain ones:
#  * routing: each token takes the k experts with the largest router logits
#    (equal logits: the lower expert index first), weighted by the softmax of
#    those k logits;
#  * w13's rows are the gate (w1) rows followed by the up (w3) rows; the
#    activation is silu(gate) * up, silu(g) = g / (1 + exp(-g)), taken in the
#    bf16 dtype the GEMM returns and quantised per token for w2;
#  * the token's output is the weighted sum of its k expert outputs.


def moe_topk(logits, k):
    """Top-k routing: for each token (row of the float32 logits [tokens, E])
    the k experts with the largest logits, largest first, equal logits taken
    in increasing expert order; weights = softmax of the selected logits
    (the softmax over all experts restricted to the k and renormalised, which
    is the same quantity), computed in float64.
    Returns (ids int32 [tokens, k], weights float64 [tokens, k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert 1 <= k <= E
    # a stable sort on the negated logits keeps equal logits in index order
    ids = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(axis=1, keepdims=True)


def moe_sort(ids, E):
    """Expert-sorted order of the routed (token, expert) pairs: sorted by
    expert, then by token. Returns (row_ids int32 [T]: the token of each sorted
    row; expert_offsets int32 [E+1]: where each expert's rows start; pos int32
    [tokens, k]: the sorted row of the pair (t, ids[t, j]))."""
    ids = np.asarray(ids, dtype=np.int64)
    tokens, k = ids.shape
    tok = np.repeat(np.arange(tokens), k)
    exp = ids.reshape(-1)
    order = np.lexsort((tok, exp))  # primary key expert, then token
    row_ids = tok[order].astype(np.int32)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(np.bincount(exp, minlength=E))
    pos = np.empty(tokens * k, np.int64)
    pos[order] = np.arange(tokens * k)
    return row_ids, offsets.astype(np.int32), pos.reshape(tokens, k).astype(np.int32)


def silu_mul_bf16(h_bits, inter):
    """The activated product of the fused w13 output h (bf16 bits [T, 2*inter]):
    gate = h[:, :inter], up = h[:, inter:], a = silu(gate) * up with
    silu(g) = g / (1 + exp(-g)), formed in float64 from the bf16 values and
    rounded once to bf16. Returns bf16 bits [T, inter]."""
    h = bf16_bits_to_f32(h_bits).astype(np.float64)
    g, u = h[:, :inter], h[:, inter:2 * inter]
    with np.errstate(over="ignore"):
        a = g / (1.0 + np.exp(-g)) * u
    return f64_to_bf16_bits(a)


def rmsnorm_bf16(x_bits, gamma_bits, eps, residual_bits=None):
    """RMS normalisation of bf16 rows [M, K] with a bf16 weight gamma [K],
    the op whose output the per-token quantiser takes in a decoder layer
    (the quantiser runs right before the GEMM, [SGLang] 핵심 코드 분석 §3):
        h = x                     (no residual), or
        h = bf16(x + residual)    (the residual add, rounded once),
        y = bf16(h * gamma / sqrt(mean_k(h**2) + eps)),
    each value formed in float64 and rounded once to bf16. The float64 sum of
    two bf16 values is exact while their exponents are within 44 of each
    other; h**2 is exact, and the mean and the quotient carry float64
    rounding only. Returns (h_bits, y_bits); h is the new residual."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    if residual_bits is not None:
        h_bits = f64_to_bf16_bits(x + bf16_bits_to_f32(residual_bits).astype(np.float64))
    else:
        h_bits = np.asarray(x_bits, dtype=np.uint16).copy()
    h = bf16_bits_to_f32(h_bits).astype(np.float64)
    g = bf16_bits_to_f32(gamma_bits).astype(np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True) if h.shape[1] else np.zeros((h.shape[0], 1))
    y = h / np.sqrt(ms + float(np.float32(eps))) * g[None, :]
    return h_bits, f64_to_bf16_bits(y)


def rmsnorm_quant(x_bits, gamma_bits, eps, residual_bits=None):
    """RMS normalisation followed by dynamic per-token symmetric quantisation
    of its bf16 output (quant_dyn_sym). Returns (h_bits, y_bits, q, s)."""
    h_bits, y_bits = rmsnorm_bf16(x_bits, gamma_bits, eps, residual_bits)
    q, s = quant_dyn_sym(y_bits)
    return h_bits, y_bits, q, s


def moe_combine(y_bits, pos, weights):
    """out[t] = sum_j weights[t, j] * y[pos[t, j]] (y: the expert outputs in
    sorted order, bf16 bits [T, N]), formed in float64 and rounded once to
    bf16. Returns bf16 bits [tokens, N]."""
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    w = np.asarray(weights, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    acc = np.zeros((pos.shape[0], y.shape[1]), np.float64)
    for j in range(pos.shape[1]):
        acc += w[:, j:j + 1] * y[pos[:, j]]
    return f64_to_bf16_bits(acc)


def moe_block(x_bits, logits, k, w13, s13, w2, s2):
    """The int8 MoE expert block, step by step: per-token symmetric
    quantisation of x [tokens, H]; top-k routing; the grouped w13 GEMM
    (w13 int8 [E, 2I, H], per-row scales s13 [E, 2I]) on each routed row;
    silu(gate) * up in bf16; per-token symmetric quantisation of that; the
    grouped w2 GEMM (w2 int8 [E, H, I], s2 [E, H]); the weighted combine.
    Returns a dict of every intermediate and the output (bf16 bits)."""
    E, two_i, H = w13.shape
    inter = two_i // 2
    xq, sx = quant_dyn_sym(x_bits)
    ids, wts = moe_topk(logits, k)
    row_ids, offsets, pos = moe_sort(ids, E)
    h, _ = grouped_scaled_mm(xq, sx, w13, s13, offsets, row_ids=row_ids)
    act = silu_mul_bf16(h, inter)
    aq, sa = quant_dyn_sym(act)
    y, _ = grouped_scaled_mm(aq, sa, w2, s2, offsets)
    out = moe_combine(y, pos, wts)
    return dict(xq=xq, sx=sx, ids=ids, weights=wts, row_ids=row_ids, offsets=offsets, pos=pos,
                h=h, act=act, aq=aq, sa=sa, y=y, out=out)


# ------------------------------------------------------------ W8A8 FP8 --
#
# The W8A8 FP8 scheme of [SGLang] 핵심 코드 분석 §1-§2: E4M3 weights and
# activations; a weight scale per channel ([N, 1]), per tensor (one per
# fused partition), or per 128 x 128 block ([N/128, K/128]); the block path
# (w8a8_block_fp8_linear) quantises the activation per token in groups of
# 128 along K, the others per token (the per-token / per-channel path) or
# with a static per-tensor input scale. Readings: the activation scale is the
# group's absmax over the largest E4M3 value (448), the FP8 counterpart of
# the int8 absmax/127 rule; an all-zero row (or group) gives scale 1; codes
# are the quotient x / s rounded to nearest E4M3 (ties to even), saturated at
# +-448; the product is exact and the scales are applied per K block before
# the block sums are added.

FP8_MAX = 448.0
FP8_ACT_TOKEN, FP8_ACT_TENSOR, FP8_ACT_GROUP128 = 0, 1, 2
FP8_W_TENSOR, FP8_W_CHANNEL, FP8_W_BLOCK128 = 0, 1, 2


def e4m3fn_encode(v):
    """Nearest OCP E4M3FN code of each float32 value (ties to the even code,
    whose last mantissa bit is 0), |v| <= 448 (larger values are outside the
    encoding's range and must be clamped first). The sign bit is kept, so -0
    and negative values that round to zero give 0x80. Found by searching the
    sorted non-negative values of e4m3fn_table()."""
    v = np.asarray(v, dtype=np.float32)
    assert not np.any(np.isnan(v)) and np.all(np.abs(v) <= FP8_MAX)
    mags = e4m3fn_table()[:127].astype(np.float64)  # codes 0 .. 126, increasing
    a = np.abs(v).astype(np.float64)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)  # first magnitude >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quant_fp8(x_bits, mode, s_in=None, group=128):
    """E4M3 quantisation of bf16 activations [M, K] ([SGLang] §1-§2).
    FP8_ACT_TOKEN:   s[t] = max_k |x_tk| / 448                 (scales [M])
    FP8_ACT_TENSOR:  s = s_in                                  (given)
    FP8_ACT_GROUP128: s[g, t] = max over k in group g |x_tk| / 448, groups of
                     128 along K (the last may be shorter)     (scales [G, M])
    An all-zero row (group) gives s = 1. q = E4M3(clamp(fl(x / s), -448, 448)).
    Returns (codes uint8 [M, K], scales float32 or None)."""
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    if mode == FP8_ACT_TENSOR:
        s_full = np.full((M, K), _F(s_in), _F)
        scales = None
    elif mode == FP8_ACT_TOKEN:
        a = np.max(np.abs(x), axis=1) if K else np.zeros(M, _F)
        scales = np.where(a == 0, _F(1), a / _F(FP8_MAX)).astype(_F)
        s_full = np.repeat(scales[:, None], K, axis=1)
    elif mode == FP8_ACT_GROUP128:
        G = -(-K // group)
        scales = np.empty((G, M), _F)
        s_full = np.empty((M, K), _F)
        for g in range(G):
            blk = x[:, g * group:(g + 1) * group]
            a = np.max(np.abs(blk), axis=1)
            scales[g] = np.where(a == 0, _F(1), a / _F(FP8_MAX)).astype(_F)
            s_full[:, g * group:(g + 1) * group] = scales[g][:, None]
    else:
        raise ValueError(f"unknown FP8 activation mode {mode}")
    with np.errstate(over="ignore"):
        t = (x / s_full).astype(_F)
    t = np.clip(t, _F(-FP8_MAX), _F(FP8_MAX))
    return e4m3fn_encode(t), scales


def scaled_mm_fp8(xq, wq, s_x, s_w, act_mode, w_mode, bias_bits=None, block=128):
    """The W8A8 FP8 GEMM ([SGLang] §2): out[t, n] = sum_k dec(xq[t, k]) *
    dec(wq[n, k]) with the scales applied, plus bias, rounded once to bf16.
    Per-tensor / per-channel weights: y = acc * s_x[t] (or s_x) * s_w[n] (or
    s_w). 128 x 128 blocks: y = sum_g acc_g * s_x[g, t] * s_w[n // 128, g],
    acc_g the sum over the K group g (activation scales group-major [G, M]).
    The products of E4M3 values are exact in float64 and so are the sums
    (at most 2^51 apart within a 128-wide group). Returns (bf16 bits [M, N],
    y float64 [M, N])."""
    dec = e4m3fn_table().astype(np.float64)
    X = dec[np.asarray(xq, np.uint8)]
    Wt = dec[np.asarray(wq, np.uint8)]
    M, K = X.shape
    N = Wt.shape[0]
    if w_mode == FP8_W_BLOCK128:
        assert act_mode == FP8_ACT_GROUP128
        sx = np.asarray(s_x, np.float32).astype(np.float64)
        sw = np.asarray(s_w, np.float32).astype(np.float64)
        y = np.zeros((M, N), np.float64)
        nblk = np.arange(N) // block
        for g in range(-(-K // block)):
            acc = X[:, g * block:(g + 1) * block] @ Wt[:, g * block:(g + 1) * block].T
            y += acc * sx[g][:, None] * sw[nblk, g][None, :]
    else:
        assert act_mode in (FP8_ACT_TOKEN, FP8_ACT_TENSOR)
        sx = np.asarray(s_x, np.float32).astype(np.float64).reshape(-1)
        sw = np.asarray(s_w, np.float32).astype(np.float64).reshape(-1)
        sx = sx[:, None] if act_mode == FP8_ACT_TOKEN else sx[0]    # [M] per token, or one scale
        sw = sw[None, :] if w_mode == FP8_W_CHANNEL else sw[0]      # [N] per channel, or one scale
        y = (X @ Wt.T) * sx * sw
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return f64_to_bf16_bits(y), y
