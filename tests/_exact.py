"""Exact rational arithmetic for pinning the oracle's floating-point decisions.

Independent of NumPy's division and float16 conversion: values are Python
Fractions and rounding to a binary format is written out from the IEEE 754
definition (round to nearest, ties to even, gradual underflow).
"""
from __future__ import annotations

from fractions import Fraction


def rne(x: Fraction, p: int, emin: int) -> Fraction:
    """Round x to the nearest value of a binary format with ``p`` significand bits
    (hidden bit included) and minimum normal exponent ``emin``; ties to even.
    No overflow handling (callers stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # e = floor(log2(a)), exactly
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                      # subnormals share the ulp of the smallest normal
    ulp = Fraction(2) ** (e - (p - 1))
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(x: Fraction) -> Fraction:
    return rne(x, 24, -126)


def f16(x: Fraction) -> Fraction:
    return rne(x, 11, -14)


def nearest_code(r: Fraction, lo: int = -127, hi: int = 127) -> int:
    """Brute force: the integer in [lo, hi] nearest to r, ties to even."""
    return min(range(lo, hi + 1), key=lambda c: (abs(r - c), c % 2))


def quant_group_exact(xs, brute: bool = False):
    """Quantise one group of float32 values exactly as the rule reads with fp32
    division: s = f16(f32(amax / 127)); code = nearest integer in [-127, 127] to
    f32(x / s) (0 when s == 0).  Returns (s as Fraction, list of codes)."""
    fx = [Fraction(float(x)) for x in xs]
    amax = max(abs(v) for v in fx)
    s = f16(f32(amax / 127))
    codes = []
    for v in fx:
        if s == 0:
            codes.append(0)
            continue
        r = f32(v / s)
        if brute:
            codes.append(nearest_code(r))
        else:
            n = r.numerator // r.denominator
            cands = [c for c in (n, n + 1) if -127 <= c <= 127] or [127 if r > 0 else -127]
            c = min(cands, key=lambda c: (abs(r - c), c % 2))
            codes.append(c)
    return s, codes


def quant_block_exact(xs, qmax: int, lo: int, hi: int, brute: bool = False):
    """The same rule for any symmetric range: s = f16(f32(amax / qmax)); code = the
    integer in [lo, hi] nearest to f32(x / s), ties to even (0 when s == 0)."""
    fx = [Fraction(float(x)) for x in xs]
    amax = max(abs(v) for v in fx)
    s = f16(f32(amax / qmax))
    codes = []
    for v in fx:
        if s == 0:
            codes.append(0)
            continue
        r = f32(v / s)
        if brute:
            codes.append(nearest_code(r, lo, hi))
        else:
            n = r.numerator // r.denominator
            cands = [c for c in (n, n + 1) if lo <= c <= hi] or [hi if r > 0 else lo]
            codes.append(min(cands, key=lambda c: (abs(r - c), c % 2)))
    return s, codes


def fwht_f32_exact(xs):
    """The butterfly Walsh-Hadamard transform with each addition and subtraction
    rounded to fp32, written out in exact fractions: stage h = 1, 2, 4, ... maps
    (y[i], y[i + h]) to (f32(y[i] + y[i + h]), f32(y[i] - y[i + h])) for i in the
    first half of each block of 2h."""
    y = [Fraction(float(v)) for v in xs]
    n = len(y)
    h = 1
    while h < n:
        for i0 in range(0, n, 2 * h):
            for i in range(i0, i0 + h):
                a, b = y[i], y[i + h]
                y[i], y[i + h] = f32(a + b), f32(a - b)
        h *= 2
    return y
