"""Exact-rational helpers for brute-force pins of the oracle (tests only)."""
from fractions import Fraction

import numpy as np


def frac(x) -> Fraction:
    """Exact value of a binary float (numpy fp32/fp64 or Python float)."""
    return Fraction(float(x))


def _round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rn32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), finite range."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    m = _round_half_even(a * Fraction(2) ** (23 - e))
    val = Fraction(m) * Fraction(2) ** (e - 23)
    return np.float32(sign * float(val))


def round_half_even(fr: Fraction) -> int:
    return _round_half_even(fr)


def nearest_exact(v: Fraction, cb) -> int:
    """argmin_i |v - cb_i| in exact arithmetic, first minimum (lower index)."""
    best, bd = 0, abs(v - frac(cb[0]))
    for i in range(1, len(cb)):
        d = abs(v - frac(cb[i]))
        if d < bd:
            best, bd = i, d
    return best
