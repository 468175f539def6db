"""Exact rational arithmetic used to pin the oracle (no floating point).

Written from the IEEE-754 definitions: a binary format with ``p`` significand
bits and minimum normal exponent ``emin`` represents ``n * 2^(e - p + 1)``;
round-to-nearest picks the representable value nearest the exact one, ties
to the even significand.
"""

from fractions import Fraction


def rne_int(v):
    """Nearest integer to Fraction v, ties to even."""
    fl = v.numerator // v.denominator
    frac = v - fl
    if frac > Fraction(1, 2):
        return fl + 1
    if frac < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_binary(v, p, emin, emax):
    """Round Fraction v to the binary format (p, emin, emax); returns Fraction
    or +-inf as float."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - p + 1)
    n = rne_int(a / quantum)
    r = n * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * float("inf")
    return sign * r


def rn16_exact(v):
    return round_binary(v, 11, -14, 15)


def rn32_exact(v):
    return round_binary(v, 24, -126, 127)


def rbf16_exact(v):
    """bfloat16: 8 significand bits, binary32's exponent range."""
    return round_binary(v, 8, -126, 127)
