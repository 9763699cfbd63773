"""Exact-rational brute force used to pin the oracle (tests only).

Independent of ``oracle/``: values are Python ``Fraction``s, and rounding is
an exhaustive search for the nearest representable value (ties to the even
code), not a midpoint comparison.
"""

from fractions import Fraction

import numpy as np


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a bf16 bit pattern from its fields."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "inf/nan not representable"
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** -126
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if s else v


def f32_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def e4m3_values():
    """All 127 finite non-negative OCP E4M3FN values by code, from the
    format's fields (sign 1, exponent 4 with bias 7, mantissa 3)."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        if e == 0:
            out.append(Fraction(m, 8) * Fraction(2) ** -6)
        else:
            out.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]
E4M3 = e4m3_values()


def nearest_even(q: Fraction, values) -> int:
    """Exhaustive nearest-value search; equal distance -> even code; values
    above the largest saturate (the largest is then the nearest anyway)."""
    best, bestd = None, None
    for c, v in enumerate(values):
        d = abs(q - v)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    return best


def quantize_block_exact(bits16, gs: Fraction):
    """Reference block quantizer in exact rationals: (nibbles[16], scale code)."""
    xs = [bf16_fraction(int(b)) for b in bits16]
    amax = max(abs(x) for x in xs)
    sb_code = nearest_even(amax / (6 * gs), E4M3)
    sb = E4M3[sb_code]
    nibs = []
    for b, x in zip(bits16, xs):
        sign = (int(b) >> 15) & 1
        if sb == 0:
            mag = 0
        else:
            mag = nearest_even(abs(x) / (sb * gs), E2M1)
        nibs.append((sign << 3) | mag)
    return nibs, sb_code


def bf16_round_exact(v: Fraction) -> int:
    """bf16 bit pattern nearest to the rational v, ties to even mantissa,
    by exhaustive comparison of the two neighbouring bf16 values."""
    s = 1 if v < 0 else 0
    a = -v if s else v
    if a == 0:
        return s << 15
    # find the binade
    e = 0
    while Fraction(2) ** e <= a:
        e += 1
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    # a in [2**(e-1), 2**e): spacing 2**(e-8), but not below 2**-133
    sp = Fraction(2) ** max(e - 8, -133)
    k = a / sp
    lo = k.numerator // k.denominator
    frac = k - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    mag = lo * sp
    if mag >= Fraction(2) ** 128:
        return (s << 15) | 0x7F80
    # encode mag
    if mag < Fraction(2) ** -126:
        m = mag / (Fraction(2) ** -133)
        assert m.denominator == 1
        return (s << 15) | int(m)
    ee = 0
    while Fraction(2) ** (ee + 1) <= mag:
        ee += 1
    while Fraction(2) ** ee > mag:
        ee -= 1
    m = (mag / Fraction(2) ** ee - 1) * 128
    assert m.denominator == 1
    return (s << 15) | ((ee + 127) << 7) | int(m)
