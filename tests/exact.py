"""Exact rational helpers used to pin the oracle (pure Python integers).

Nothing here shares code with the oracle: values are decoded from their bit
patterns and rounded to IEEE binary32 with integer arithmetic, so that
agreement with the oracle's float arithmetic is evidence, not a tautology.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def f32_to_fraction(v: float) -> Fraction:
    """Exact value of a finite binary32 (given as a Python float holding it)."""
    b = f32_bits(v)
    sign = -1 if b >> 31 else 1
    e = (b >> 23) & 0xFF
    f = b & 0x7FFFFF
    if e == 0:
        m, ex = f, -149
    elif e == 255:
        raise ValueError("non-finite")
    else:
        m, ex = (1 << 23) | f, e - 150
    return sign * Fraction(m) * (Fraction(2) ** ex)


def half_bits_to_fraction(h: int) -> Fraction:
    sign = -1 if (h >> 15) & 1 else 1
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 31:
        raise ValueError("non-finite")
    if e == 0:
        return sign * Fraction(f) * (Fraction(2) ** -24)
    return sign * Fraction(1024 + f) * (Fraction(2) ** (e - 25))


def bf16_bits_to_fraction(b: int) -> Fraction:
    return f32_to_fraction(bits_f32(b << 16))


def _rne_div(num: int, den: int) -> int:
    """round(num / den) to nearest, ties to even, for num >= 0, den > 0."""
    q, r = divmod(num, den)
    if 2 * r > den or (2 * r == den and q & 1):
        q += 1
    return q


def fraction_to_f32_bits(x: Fraction) -> int:
    """Round a rational to binary32, nearest-even, gradual underflow."""
    if x == 0:
        return 0
    sign = 0
    if x < 0:
        sign, x = 1, -x
    num, den = x.numerator, x.denominator
    # e such that 2^e <= x < 2^(e+1)
    e = num.bit_length() - den.bit_length()
    if Fraction(num, den) < Fraction(2) ** e:
        e -= 1
    lsb = max(e - 23, -149)
    # m = round(x / 2^lsb)
    if lsb >= 0:
        m = _rne_div(num, den << lsb)
    else:
        m = _rne_div(num << (-lsb), den)
    if m == 0:
        return sign << 31
    if m >= (1 << 24):  # carried into the next binade
        m >>= 1
        lsb += 1
    if m < (1 << 23):  # subnormal
        assert lsb == -149
        return (sign << 31) | m
    biased = lsb + 150
    if biased >= 255:
        return (sign << 31) | 0x7F800000
    return (sign << 31) | (biased << 23) | (m - (1 << 23))


def rne_to_int(x: Fraction) -> int:
    """Nearest integer, ties to even."""
    neg = x < 0
    a = -x if neg else x
    q = _rne_div(a.numerator, a.denominator)
    return -q if neg else q


def quant_code_exact(x: Fraction, scale_bits: int) -> int:
    """clamp(rne(fl32(x / scale)), -127, 127) with the quotient rounded exactly."""
    sc = f32_to_fraction(bits_f32(scale_bits))
    if sc == 0:
        return 0
    r = f32_to_fraction(bits_f32(fraction_to_f32_bits(x / sc)))
    return max(-127, min(127, rne_to_int(r)))


def quant_scale_exact(absmax: Fraction) -> int:
    return fraction_to_f32_bits(absmax / 127)
