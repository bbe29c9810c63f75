"""Exact-rational brute force used to pin the oracle (tests only).

Nothing here shares code with ``oracle/``: values are rebuilt from the
format definitions with ``fractions.Fraction`` and nearest points are found
by exhaustive search over the whole representable set.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def f32_exact(v) -> Fraction:
    """Exact rational value of a binary32 number (finite)."""
    return Fraction(float(np.float32(v)))


def e4m3_all_finite_nonneg():
    """[(code, Fraction value)] for the 127 finite non-negative E4M3 bytes,
    built from the bit layout (4 exponent bits, bias 7, 3 mantissa bits)."""
    out = []
    for code in range(0x7F):
        E, m = code >> 3, code & 7
        if E == 0:
            val = Fraction(m, 8) * Fraction(1, 2 ** 6)
        else:
            val = (1 + Fraction(m, 8)) * (Fraction(2) ** (E - 7))
        out.append((code, val))
    return out


def e2m1_all_nonneg():
    """[(code, Fraction value)] for the 8 E2M1 magnitudes, from the bit
    layout (2 exponent bits, bias 1, 1 mantissa bit; exponent 0 subnormal)."""
    out = []
    for code in range(8):
        E, m = code >> 1, code & 1
        if E == 0:
            val = Fraction(m, 2)
        else:
            val = (1 + Fraction(m, 2)) * (Fraction(2) ** (E - 1))
        out.append((code, val))
    return out


def nearest_code(t: Fraction, table):
    """Exhaustive nearest; ties to the even code; above the top -> top."""
    best = None
    for code, val in table:
        d = abs(t - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def nearest_bf16(v: Fraction) -> Fraction:
    """Nearest bfloat16 value to v (ties to even), finite range only."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** max(e - 7, -133)   # quantum of bf16 at that binade
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * q
