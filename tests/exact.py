"""Exact-arithmetic helpers for pinning floating-point steps of the oracle.

Rationals (``fractions.Fraction``) rounded once to the nearest fp32, ties to
even, by a routine written from the IEEE 754 binary32 format alone: 24-bit
significand, exponent range [-126, 127], subnormal quantum 2^-149.
"""
from fractions import Fraction

import numpy as np


def round_to_f32(q: Fraction) -> np.float32:
    """The fp32 nearest to the rational ``q``, ties to even (one rounding)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormals share the quantum 2^-149
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum                       # significand in units of the quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * quantum
    if val >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))      # exact: val is representable in fp32
        assert Fraction(float(out)) == val
    return np.float32(-out) if neg else out


def f(x) -> Fraction:
    """The exact rational value of a finite fp32/fp64 number."""
    return Fraction(float(x))


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def _f32_neighbours(c: np.float32):
    return (np.nextafter(c, np.float32(-np.inf), dtype=np.float32), c,
            np.nextafter(c, np.float32(np.inf), dtype=np.float32))


def round_sqrt_f32(q: Fraction) -> np.float32:
    """The fp32 nearest to sqrt(q) for a rational q >= 0 (correct rounding),
    found by bracketing sqrt(q) between the exact midpoints of fp32
    neighbours: c is the answer iff mid(c-, c)^2 <= q <= mid(c, c+)^2."""
    if q == 0:
        return np.float32(0.0)
    c = np.float32(np.sqrt(float(q)))
    for _ in range(4):
        lo_n, _, hi_n = _f32_neighbours(c)
        lo = (f(lo_n) + f(c)) / 2
        hi = (f(c) + f(hi_n)) / 2
        if lo * lo <= q <= hi * hi:
            assert lo * lo != q and hi * hi != q, "tie"
            return c
        c = lo_n if q < lo * lo else hi_n
    raise AssertionError("no fp32 bracket found")
