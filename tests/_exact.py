"""Exact-rational brute force used to pin the oracle codec (tests only).

Independent of ``oracle/``: every quotient is formed exactly with
``fractions.Fraction`` and the nearest grid value is found by scanning the
whole grid, so a mistake in the oracle's divide-free comparisons, tie rule or
vectorisation shows up as a mismatch.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _e4m3_fraction(code: int):
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 64)
    return (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


E4M3_POS_FR = [_e4m3_fraction(c) for c in range(127)]
E2M1_POS_FR = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
               Fraction(4), Fraction(6)]


def nearest_code(value: Fraction, grid) -> int:
    """Index of the grid value nearest to ``value`` (>= 0), ties to the even index."""
    best = None
    best_d = None
    for i, g in enumerate(grid):
        d = abs(value - g)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def e4m3_code(value: Fraction, negative: bool = False) -> int:
    return nearest_code(abs(value), E4M3_POS_FR) | (0x80 if negative else 0)


def fp4_group(xs) -> tuple[list[int], int]:
    """(16 four-bit codes, scale byte) of one group of fp32 values."""
    fr = [Fraction(float(x)) for x in xs]
    amax = max(abs(f) for f in fr)
    sc = nearest_code(amax / 6, E4M3_POS_FR)
    s = E4M3_POS_FR[sc]
    codes = []
    for x, f in zip(xs, fr):
        neg = math.copysign(1.0, float(x)) < 0
        mag = 0 if s == 0 else nearest_code(abs(f) / s, E2M1_POS_FR)
        codes.append(mag | (8 if neg else 0))
    return codes, sc


def fraction_to_f32(v: Fraction) -> float:
    """Correctly rounded (ties to even) fp32 value of a rational, finite range only."""
    if v == 0:
        return 0.0
    neg = v < 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)); fp32 keeps 24 significant bits (subnormals: fixed 2^-149 step)
    step_exp = max(e - 23, -149)
    q = a / (Fraction(2) ** step_exp)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    out = float(n) * 2.0 ** step_exp
    return float(np.float32(-out if neg else out))


def fp8_row(xs) -> tuple[list[int], float]:
    """(E4M3 codes, fp32 row scale) of one window row of fp32 values."""
    fr = [Fraction(float(x)) for x in xs]
    amax = max(abs(f) for f in fr)
    r = 1.0 if amax == 0 else fraction_to_f32(amax / 448)
    codes = []
    for x, f in zip(xs, fr):
        y = fraction_to_f32(f / Fraction(r))
        codes.append(e4m3_code(Fraction(y), math.copysign(1.0, y) < 0 or (y == 0 and math.copysign(1.0, float(x)) < 0)))
    return codes, r
