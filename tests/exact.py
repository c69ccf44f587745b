"""Exact-arithmetic helpers for the oracle pins (pure Python integers and
Fractions; independent of numpy's floating point)."""
from __future__ import annotations

import struct
from fractions import Fraction


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def round_to_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest IEEE binary32 value, ties to even,
    with gradual underflow.  Written from the format's definition: 24-bit
    significand, minimum normal exponent -126, subnormal spacing 2**-149."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    # e = floor(log2(a))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # subnormals share the minimum exponent
    scaled = a * Fraction(2) ** (23 - e)  # significand in units of the last place
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    if m == 1 << 24:                      # carried into the next binade
        m >>= 1
        e += 1
    if e > 127:
        raise OverflowError
    return sign * float(Fraction(m) * Fraction(2) ** (e - 23))


def rne_int(q: Fraction) -> int:
    """Nearest integer to an exact rational, ties to even."""
    f = q.numerator // q.denominator
    rem = q - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def round_to_bf16(q: Fraction) -> float:
    """Round an exact rational to the nearest bfloat16 value, ties to even, with
    gradual underflow.  From the format's definition: 8-bit significand (7
    stored bits), the binary32 exponent range (minimum normal exponent -126),
    subnormal spacing 2**-133."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    scaled = a * Fraction(2) ** (7 - e)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    if m == 1 << 8:
        m >>= 1
        e += 1
    if e > 127:
        raise OverflowError
    return sign * float(Fraction(m) * Fraction(2) ** (e - 7))
