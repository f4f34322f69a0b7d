"""Exact-arithmetic helpers for pinning floating-point steps of the oracle.

Rationals (``fractions.Fraction``) rounded once to the nearest fp32 or bf16,
ties to even, by a routine written from the formats alone: 24 (fp32) or 8
(bf16) significant bits, exponent range [-126, 127], subnormal quantum
2^-149 (fp32) or 2^-133 (bf16).
"""
from fractions import Fraction

import numpy as np


def _round_binary(a: Fraction, p: int) -> Fraction:
    """The value with p significant bits nearest to a > 0, ties to even, in
    a format whose smallest normal is 2^-126 (fp32 and bf16 share it; below
    it the spacing stays that of the binade [2^-126, 2^-125))."""
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - (p - 1))
    m = a / quantum                       # significand in units of the quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * quantum


def round_to_f32(q: Fraction) -> np.float32:
    """The fp32 nearest to the rational ``q``, ties to even (one rounding)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    val = _round_binary(-q if neg else q, 24)
    if val >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))      # exact: val is representable in fp32
        assert Fraction(float(out)) == val
    return np.float32(-out) if neg else out


def round_to_bf16(q: Fraction) -> np.uint16:
    """The bits of the bf16 nearest to the rational ``q``, ties to even (one
    rounding; 8 significant bits, fp32's exponent range)."""
    if q == 0:
        return np.uint16(0)
    neg = q < 0
    val = _round_binary(-q if neg else q, 8)
    if val >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        f32 = np.float32(float(val))
        assert Fraction(float(f32)) == val
        u = int(f32.view(np.uint32))
        assert u & 0xFFFF == 0
        bits = u >> 16
    return np.uint16(bits | (0x8000 if neg else 0))


def bf16_midpoint_near(x: float, bound: float) -> bool:
    """Whether a rounding midpoint between two bf16 neighbours lies within
    ``bound`` of x (then a value within ``bound`` of x may round to either)."""
    lo = round_to_bf16(Fraction(x) - Fraction(bound))
    hi = round_to_bf16(Fraction(x) + Fraction(bound))
    return lo != hi


def f32_midpoint_near(x: float, bound: float) -> bool:
    """The same for fp32 rounding midpoints."""
    return round_to_f32(Fraction(x) - Fraction(bound)) != round_to_f32(Fraction(x) + Fraction(bound))


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
