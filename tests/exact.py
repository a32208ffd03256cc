"""Exact rational arithmetic for pinning the oracle's floating point.

IEEE-754 defines each basic operation as the exact real result rounded to the
destination format.  This module computes that directly: values are Python
Fractions, and `round_binary` rounds a rational to the nearest number of a
binary format with p significand bits and minimum normal exponent emin,
ties to the even significand, overflowing to infinity.  It uses neither the
host's float unit nor numpy's, so agreement with the oracle is evidence about
the oracle rather than a restatement of it.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

INF = float("inf")


def _floor_log2(x: Fraction) -> int:
    """e with 2^e <= x < 2^(e+1), for x > 0."""
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    # adjust: compare x with 2^e
    if e >= 0:
        if n < d << e:
            e -= 1
    else:
        if n << (-e) < d:
            e -= 1
    return e


def round_binary(x: Fraction, p: int, emin: int, emax: int):
    """Round x to the format (p, emin, emax), nearest-even.  Returns a Fraction
    or +-INF.  Zero returns Fraction(0) (the sign of zero is tracked by the
    caller where it matters)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    qe = e - (p - 1)  # exponent of the last significand bit
    scaled = a / Fraction(2) ** qe if qe >= 0 else a * (1 << (-qe))
    r = math.floor(scaled)
    rem = scaled - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = Fraction(r) * (Fraction(2) ** qe)
    if val >= Fraction(2) ** (emax + 1):
        return sign * INF
    return sign * val


def f32(x: Fraction):
    return round_binary(x, 24, -126, 127)


def bf16(x: Fraction):
    return round_binary(x, 8, -126, 127)


def frac(v) -> Fraction:
    """Exact value of a finite float / np.float32."""
    return Fraction(float(v))


def f32_bits_of(x) -> int:
    """Bit pattern of the binary32 number equal to the (already representable) x."""
    if isinstance(x, float) and math.isinf(x):
        return 0x7F800000 if x > 0 else 0xFF800000
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bf16_bits_of(x, negative_zero: bool = False) -> int:
    """Bit pattern of the bfloat16 number equal to x (x representable in bf16)."""
    if x == 0:
        return 0x8000 if negative_zero else 0x0000
    u = f32_bits_of(x)
    assert u & 0xFFFF == 0, "value is not a bfloat16 number"
    return u >> 16


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def ulp_distance_bf16(a: int, b: int) -> int:
    """Distance in bf16 spacings between two finite bf16 bit patterns
    (+0 and -0 are the same point)."""
    def key(h):
        h &= 0xFFFF
        return -(h & 0x7FFF) if h & 0x8000 else h
    return abs(key(a) - key(b))
