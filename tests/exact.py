"""Exact rational arithmetic used to pin the oracle by brute force.

Everything here is written from the IEEE-754 definitions with Python's
``fractions.Fraction`` and touches neither numpy's float32 ops nor the oracle,
so a mistake in either (a multiply by a reciprocal instead of a division, a
round-half-away-from-zero, a wrong clamp) shows up as a mismatch.
"""

from __future__ import annotations

import struct
from fractions import Fraction


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bf16_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "finite values only"
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** (1 - 127)
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def f32_to_fraction(v: float) -> Fraction:
    return Fraction(v)  # a binary32 value is exactly representable in a double


def round_half_even(fr: Fraction) -> int:
    """Nearest integer, ties to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def nearest_f32(fr: Fraction) -> Fraction:
    """Correctly rounded binary32 value of an exact rational (ties to even).

    Normal numbers keep 24 significant bits; below 2**-126 the spacing is
    2**-149. Overflow is not handled (not reached by the callers).
    """
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e - 23, -149)
    quantum = Fraction(2) ** q_exp
    n = round_half_even(a / quantum)
    return sign * n * quantum


def nearest_bf16(fr: Fraction) -> Fraction:
    """Correctly rounded bf16 value of an exact rational (ties to even): 8
    significant bits, spacing 2**-133 below 2**-126. Overflow is not handled."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 7, -133)
    return sign * round_half_even(a / quantum) * quantum


def clamp(v: int, lo: int, hi: int) -> int:
    return lo if v < lo else hi if v > hi else v


# ---------------------------------------------------- vectorised exact checks

def _next_f32(v, direction):
    import numpy as np
    return np.nextafter(v.astype(np.float32), np.float32(direction * np.inf)).astype(np.float32)


def correctly_rounded_quotients(x, s):
    """Return the binary32 quotients x/s after proving, element by element and
    in exact arithmetic, that each is the correctly rounded (ties-to-even)
    value: q*s - x is computed exactly in float64 (24 + 24 significant bits
    fit in 53) for q and its two binary32 neighbours, and q must be nearest,
    taking the even significand on a tie. Raises AssertionError otherwise."""
    import numpy as np
    x = np.asarray(x, np.float32)
    s = np.asarray(s, np.float32)
    q = (x / s).astype(np.float32)
    x64, s64 = x.astype(np.float64), s.astype(np.float64)
    r0 = np.abs(q.astype(np.float64) * s64 - x64)
    for d in (-1, 1):
        nb = _next_f32(q, d)
        r1 = np.abs(nb.astype(np.float64) * s64 - x64)
        assert np.all(r0 <= r1), "a neighbour is nearer: quotient not correctly rounded"
        tie = r0 == r1
        if np.any(tie):
            even = (q.view(np.uint32) & 1) == 0
            assert np.all(even[tie]), "tie not resolved to even"
    return q


def round_half_even_array(v):
    """Round-half-to-even of float values written with floor and a comparison,
    independent of numpy's rint."""
    import numpy as np
    v = np.asarray(v, np.float64)
    f = np.floor(v)
    frac = v - f
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(f, 2) == 1))
    return (f + up).astype(np.int64)
