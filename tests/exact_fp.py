"""Exact rational arithmetic for IEEE binary32 results (test helper).

Every fp32 operation the quantizers and the dequantization perform is "the
exact result, rounded once to the nearest float32, ties to even".  These
helpers compute that from the definition with Python's exact fractions, so a
golden value derived with them depends on neither the oracle nor any
floating-point unit.  Normal-range values only (every case here stays far
from the subnormal range and from overflow).
"""
from fractions import Fraction as F

import numpy as np


def fr(x) -> F:
    """The exact value of a float32 (or of a Python float that is one)."""
    return F(float(np.float32(x)))


def rn32(v: F) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "normal range only"
    m = a / F(2) ** (e - 23)
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > F(1, 2) or (rem == F(1, 2) and mi % 2 == 1):
        mi += 1
    return np.float32(float(sign * mi * F(2) ** (e - 23)))


def rne_int(v: F) -> int:
    """Round an exact rational to the nearest integer, ties to even."""
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def div32(a, b) -> np.float32:
    """fl(a / b): the correctly rounded fp32 quotient."""
    return rn32(fr(a) / fr(b))


def mul32(a, b) -> np.float32:
    return rn32(fr(a) * fr(b))


def add32(a, b) -> np.float32:
    return rn32(fr(a) + fr(b))


def sub32(a, b) -> np.float32:
    return rn32(fr(a) - fr(b))


def clamp(q: int, lo: int, hi: int) -> int:
    return max(lo, min(hi, q))


def is_pow2(x) -> bool:
    m, _ = np.frexp(np.float32(abs(x)))
    return m == 0.5


def h(x) -> str:
    """Exact hexadecimal text of a float32 (float.fromhex reads it back)."""
    return float(np.float32(x)).hex()


def unh(s: str) -> np.float32:
    v = float.fromhex(s)
    assert float(np.float32(v)) == v, s
    return np.float32(v)
