"""Exact rational arithmetic used to pin the oracle (tests only).

Rounding of an exact rational to binary floating point, written from the
IEEE 754 definition (round to nearest, ties to even), independent of NumPy's
and the C library's float arithmetic.
"""
from fractions import Fraction
import math


def _round_fraction(fr: Fraction, mant_bits: int, min_exp: int, max_exp: int) -> Fraction:
    """Nearest value with ``mant_bits`` significant bits; subnormal quantum 2**min_exp.

    Returns a Fraction, or +-inf as a float when the rounded value overflows
    (exponent beyond ``max_exp``).
    """
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    q_exp = max(e - (mant_bits - 1), min_exp)
    scaled = a / Fraction(2) ** q_exp
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** q_exp
    if val >= Fraction(2) ** (max_exp + 1):
        return sign * math.inf
    return sign * val


def round_f32(fr: Fraction) -> float:
    r = _round_fraction(Fraction(fr), 24, -149, 127)
    return float(r)


def round_f64(fr: Fraction) -> float:
    r = _round_fraction(Fraction(fr), 53, -1074, 1023)
    return float(r)


def round_bf16(fr: Fraction) -> float:
    r = _round_fraction(Fraction(fr), 8, -133, 127)
    return float(r)


def round_half_even(fr: Fraction) -> int:
    n = math.floor(fr)
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return int(n)
