"""Exact-arithmetic helpers for pinning the oracle (independent of it).

Everything here works on Python integers and ``fractions.Fraction``: no fp32
hardware arithmetic is used, so these helpers are a second route to the
values the oracle computes with fp32 operations.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f32_bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).reshape(()).view(np.uint32))


def f32_from_bits(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def frac_of_f32(v) -> Fraction:
    """The exact rational value of a finite fp32 number."""
    b = f32_bits(v)
    sign = -1 if b >> 31 else 1
    e = (b >> 23) & 0xFF
    m = b & 0x7FFFFF
    if e == 255:
        raise ValueError("not finite")
    if e == 0:
        val = Fraction(m, 1 << 149)
    else:
        val = Fraction(m | 0x800000) * (Fraction(2) ** (e - 150))
    return sign * val


def round_half_even(q: Fraction) -> int:
    """The integer nearest to q, ties to the even integer."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_f32(q: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 value of a rational.
    Overflow is not handled (callers stay far below 2^128)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    # quantum: 2^(e-23) for normal numbers, 2^-149 in the subnormal range
    qexp = max(e - 23, -149)
    n = round_half_even(a / (Fraction(2) ** qexp))
    val = Fraction(n) * (Fraction(2) ** qexp)
    return np.float32(sign * float(val))  # val has <= 24 significant bits: exact in fp32
