"""The activation quantizers form fl(x / s) without a division:

    rs = fl(1 / s),  q = fl(x * rs),  r = fma(-q, s, x),  fl(x / s) = fma(r, rs, q)

(Markstein's theorem for round-to-nearest).  The int8 codes depend on that
quotient through round-half-to-even, so the identity must hold exactly, ties
included.  This checks it in exact rational arithmetic on scales of many
exponents and mantissa patterns (all-ones mantissas included) and on
quotients that sit on, and one ulp either side of, the ties k + 1/2.
"""
from fractions import Fraction as F

import numpy as np


def rn32(fr: F) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even (normal range)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    m = a / F(2) ** (e - 23)
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > F(1, 2) or (rem == F(1, 2) and mi % 2 == 1):
        mi += 1
    return np.float32(float(sign * mi * F(2) ** (e - 23)))


def f32(bits: int) -> np.float32:
    return np.frombuffer(np.uint32(bits).tobytes(), np.float32)[0]


def test_rn32_matches_numpy_rounding():
    rng = np.random.default_rng(3)
    for x in rng.standard_normal(2000) * 10.0 ** rng.integers(-20, 20, 2000):
        assert rn32(F(float(x))) == np.float32(x)


def test_quotient_without_division_is_correctly_rounded():
    rng = np.random.default_rng(20251014)
    checked = 0
    for trial in range(6000):
        kind = trial % 4
        if kind == 0:
            s = np.float32(rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-60, 60)))
        elif kind == 1:
            s = f32((int(rng.integers(40, 200)) << 23) | 0x7FFFFF)
        elif kind == 2:
            s = f32((int(rng.integers(40, 200)) << 23) | int(rng.integers(0, 1 << 23)))
        else:
            s = np.float32(np.float32(rng.uniform(0.1, 100.0)) / np.float32(127.0))
        k = int(rng.integers(-128, 128))
        tie = rn32((k + F(1, 2)) * F(float(s)))
        cands = [tie, np.nextafter(tie, np.float32(np.inf)), np.nextafter(tie, np.float32(-np.inf)),
                 np.float32(rng.uniform(-127.5, 127.5)) * s]
        fs = F(float(s))
        rs = rn32(1 / fs)
        frs = F(float(rs))
        for v in cands:
            fv = F(float(np.float32(v)))
            q = rn32(fv * frs)
            r = rn32(fv - fs * F(float(q)))
            got = rn32(F(float(q)) + F(float(r)) * frs)
            assert got == rn32(fv / fs), (float(v), float(s))
            checked += 1
    assert checked == 24000


def rn32_any(fr: F) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even, including
    the subnormal range (quantum 2^-149)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    q = F(2) ** (max(e, -126) - 23)
    m = a / q
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > F(1, 2) or (rem == F(1, 2) and mi % 2 == 1):
        mi += 1
    return np.float32(float(sign * mi * q))


def test_rn32_any_matches_numpy_rounding_subnormal():
    rng = np.random.default_rng(5)
    for x in rng.standard_normal(2000) * 10.0 ** rng.integers(-46, -36, 2000):
        assert rn32_any(F(float(x))) == np.float32(x)


def test_tiny_scales_by_exact_rescaling():
    """Scales below 2^-64, down to subnormal ones: x and s are both multiplied
    by 2^100 (exact: s * 2^100 < 2^36 and |x| <= 127.5 s < 2^-57), which keeps
    the real quotient and brings s into the range where the identity above
    holds; the rescaled division-free quotient equals fl(x / s)."""
    rng = np.random.default_rng(77)
    pre = F(2) ** 100
    checked = 0
    for trial in range(3000):
        kind = trial % 3
        if kind == 0:
            s = f32(int(rng.integers(1, 1 << 23)))                        # subnormal
        elif kind == 1:
            s = f32((int(rng.integers(1, 63)) << 23) | int(rng.integers(0, 1 << 23)))
        else:
            s = f32((int(rng.integers(1, 63)) << 23) | 0x7FFFFF)          # all-ones mantissa
        assert 0 < s < np.float32(2.0 ** -64)
        fs = F(float(s))
        k = int(rng.integers(-128, 128))
        tie = rn32_any((k + F(1, 2)) * fs)
        cands = [tie, np.nextafter(tie, np.float32(np.inf)), np.nextafter(tie, np.float32(-np.inf)),
                 rn32_any(F(float(rng.uniform(-127.5, 127.5))) * fs), f32(int(rng.integers(1, 64)))]
        ss = fs * pre
        assert F(float(np.float32(float(ss)))) == ss               # s * 2^100 is a float32
        rs = F(float(rn32(1 / ss)))
        for v in cands:
            fv = F(float(np.float32(v)))
            xs = fv * pre
            assert F(float(np.float32(float(xs)))) == xs           # x * 2^100 is a float32
            q = F(float(rn32_any(xs * rs)))
            r = F(float(rn32_any(xs - ss * q)))
            got = rn32_any(q + r * rs)
            assert got == rn32_any(fv / fs), (float(v), float(s))
            checked += 1
    assert checked == 15000
