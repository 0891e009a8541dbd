"""Exact-rational helpers for pinning the oracle (test-only).

Independent of oracle/: rounding is done on Python Fractions, with ties to
even via Fraction.__round__ (banker's rounding).
"""
from fractions import Fraction
import math


def _round_binary(fr: Fraction, mant_bits: int, emin: int, emax: int):
    """Round a rational to the nearest binary float with ``mant_bits``
    significant bits, minimum normal exponent ``emin`` and maximum exponent
    ``emax``; ties to even. Returns a Fraction or +-inf (float)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    unit = Fraction(2) ** (max(e, emin) - (mant_bits - 1))
    n = round(a / unit)  # ties to even
    v = n * unit
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * v


def to_f32(fr):
    return _round_binary(Fraction(fr), 24, -126, 127)


def to_f16(fr):
    return _round_binary(Fraction(fr), 11, -14, 15)


def to_bf16(fr):
    return _round_binary(Fraction(fr), 8, -126, 127)
