"""Exact-arithmetic helpers for the oracle's pins (rational numbers and
high-precision decimals, rounded once to fp32).  Independent of the oracle
and of the HIP library."""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np


def nearest_f32(q: Fraction) -> np.float32:
    """The fp32 value nearest to the exact rational q (ties to even)."""
    f = np.float32(float(q))  # within one fp32 ulp of the answer
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    best, best_d = None, None
    for c in (lo, f, hi):
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        if best is None or d < best_d or (d == best_d and int(c.view(np.uint32)) % 2 == 0):
            best, best_d = c, d
    return np.float32(best)


def exp_f32(L: float, digits: int = 60) -> np.float32:
    """RN32(e^L) from a 60-digit decimal evaluation."""
    with localcontext() as ctx:
        ctx.prec = digits
        v = Decimal(float(L)).exp()
    return nearest_f32(Fraction(v))


def ln_f32(r: float, digits: int = 60) -> np.float32:
    """RN32(ln r) from a 60-digit decimal evaluation."""
    with localcontext() as ctx:
        ctx.prec = digits
        v = Decimal(float(r)).ln()
    return nearest_f32(Fraction(v))


def normalize_f32(x: int, mean: float, std: float) -> np.float32:
    """RN32((x/255 - mean)/std), exactly, for fp32 mean and std."""
    q = (Fraction(int(x), 255) - Fraction(float(np.float32(mean)))) / Fraction(float(np.float32(std)))
    return nearest_f32(q)


def normalize_lut(mean, std) -> np.ndarray:
    """(256, C) table of the exact normalized fp32 values."""
    C = len(mean)
    return np.array([[normalize_f32(x, mean[c], std[c]) for c in range(C)] for x in range(256)],
                    dtype=np.float32)


def nearest_f64(q: Fraction) -> float:
    """The double nearest to q (CPython's int / int division rounds
    correctly, ties to even)."""
    return q.numerator / q.denominator


def sqrt_exact(q: Fraction, digits: int = 60) -> Fraction:
    """sqrt(q) to `digits` significant digits (far more than any rounding
    below needs; the square root of a float is never a rounding midpoint of
    fp32 or fp64, so the nearest value is decided by these digits)."""
    with localcontext() as ctx:
        ctx.prec = digits
        v = (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
    return Fraction(v)


def sqrt_f32(q: Fraction) -> np.float32:
    """RN32(sqrt(q))."""
    return nearest_f32(sqrt_exact(q))


def round_half_away(q: Fraction) -> int:
    """Nearest integer to q >= 0, halves away from zero."""
    return int((q + Fraction(1, 2)).__floor__())
