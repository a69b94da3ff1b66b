"""Exact rational rounding, used to pin the oracle's float arithmetic.

Independent of the oracle: values are Python Fractions and rounding to a
binary format is done from its definition (round half to even on the grid
of the value's binade, with a fixed subnormal quantum below the smallest
normal).
"""

import math
import struct
from fractions import Fraction


def round_binary(q, frac_bits, emin):
    """Round a Fraction to a binary float with ``frac_bits`` stored fraction
    bits and smallest normal exponent ``emin`` (no overflow handling).
    Returns the rounded value as a Fraction (sign kept)."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - frac_bits)
    r = round(a / quantum) * quantum  # Fraction.__round__ is half-to-even
    return r if q > 0 else -r


def to_f32_bits(q):
    r = round_binary(q, 23, -126)
    return struct.unpack("<I", struct.pack("<f", float(r)))[0] | (0x80000000 if q < 0 and r == 0 else 0)


def to_bf16_bits(q):
    r = round_binary(q, 7, -126)
    bits = struct.unpack("<I", struct.pack("<f", float(r)))[0] >> 16
    return bits


def near_tie(q, frac_bits, emin, rel=2.0 ** -40):
    """True when q lies within ``rel`` (relative) of a rounding midpoint."""
    q = Fraction(q)
    if q == 0:
        return False
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - frac_bits)
    pos = a / quantum
    frac = pos - math.floor(pos)
    return abs(frac - Fraction(1, 2)) * quantum < a * Fraction(rel)


def f32_bits_of(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]
