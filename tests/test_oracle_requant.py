"""Pins of the oracle's Q31 requantize (MCU conv front-end page,
news.rkmt.cn/news/16638, §2.3).

Besides the hand-worked table, every random case is checked against the
specification the shift-and-add implements -- round x*M/2^shift to the nearest
integer with exact halves going up, then saturate -- using exact rational
arithmetic, not the 64-bit add-and-shift itself.
"""
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden


def _spec(x, M, s):
    v = Fraction(x * M, 2 ** s)
    lo = v - Fraction(1, 2)
    # the unique integer y with v - 1/2 < y <= v + 1/2 ... ties (v = y - 1/2)
    # go up, so y is the integer in the half-open interval (v - 1/2, v + 1/2]
    y = lo.numerator // lo.denominator + 1  # smallest integer strictly above v - 1/2
    assert v - Fraction(1, 2) < y <= v + Fraction(1, 2)
    return max(-128, min(127, y))


def test_hand_table(orc):
    rows = read_golden("requant_hand_table.txt")
    assert len(rows) >= 30
    for acc, bias, M, s, want in rows:
        got = orc.requant(int(acc), int(bias), int(M), int(s))
        assert got == int(want), (acc, bias, M, s)


def test_hand_table_agrees_with_spec():
    for acc, bias, M, s, want in read_golden("requant_hand_table.txt"):
        assert _spec(int(acc) + int(bias), int(M), int(s)) == int(want)


def test_random_against_rational_spec(orc):
    g = np.random.default_rng(7)
    n = 40000
    xs = g.integers(-2 ** 31, 2 ** 31, size=n, dtype=np.int64)
    # mix full-range x with accumulator-sized x
    xs[: n // 2] = g.integers(-2 ** 24, 2 ** 24, size=n // 2)
    Ms = g.integers(0, 2 ** 31, size=n, dtype=np.int64)
    ss = g.integers(1, 64, size=n, dtype=np.int64)
    # near-saturation and tie-heavy cases
    ss[: n // 4] = g.integers(28, 46, size=n // 4)
    for x, M, s in zip(xs.tolist(), Ms.tolist(), ss.tolist()):
        assert orc.requant(x, 0, M, s) == _spec(x, M, s), (x, M, s)


def test_million_against_bigint(orc):
    """10^6 random cases (full-range x and M, every shift, plus the extremes)
    against the rounding written with Python integers, whose floor division
    does not depend on C's 64-bit arithmetic: y = floor((x M + 2^(s-1)) / 2^s),
    saturated."""
    g = np.random.default_rng(17)
    n = 1_000_000
    x = g.integers(-2 ** 31, 2 ** 31, size=n, dtype=np.int64)
    x[: n // 2] = g.integers(-2 ** 26, 2 ** 26, size=n // 2)
    M = g.integers(0, 2 ** 31, size=n, dtype=np.int64)
    s = g.integers(1, 64, size=n, dtype=np.int64)
    s[: n // 3] = g.integers(28, 46, size=n // 3)
    ext = [(xv, mv, sv) for xv in (2 ** 31 - 1, -2 ** 31, 0, 1, -1)
           for mv in (2 ** 31 - 1, 2 ** 30, 0) for sv in (1, 31, 44, 63)]
    x[: len(ext)] = [e[0] for e in ext]
    M[: len(ext)] = [e[1] for e in ext]
    s[: len(ext)] = [e[2] for e in ext]
    got = orc.requant_many(x, np.zeros(n, np.int32), M.astype(np.int32), s.astype(np.int32))
    want = [max(-128, min(127, (xi * mi + (1 << (si - 1))) >> si))
            for xi, mi, si in zip(x.tolist(), M.tolist(), s.tolist())]
    assert np.array_equal(got, np.array(want, np.int8))


def test_exact_ties_round_up(orc):
    # x*M/2^s = k + 1/2 exactly for k in a range: result must be k + 1
    s = 35
    M = 2 ** 30
    for k in range(-130, 130):
        x = (2 * k + 1) * 2 ** (s - 31)  # x*M/2^s = (2k+1)/2
        want = max(-128, min(127, k + 1))
        assert orc.requant(x, 0, M, s) == want, k


def test_identity_multiplier(orc):
    # M = 2^30, shift = 30 multiplies by exactly 1: the result is clamp(x)
    for x in range(-400, 400, 7):
        assert orc.requant(x, 0, 2 ** 30, 30) == max(-128, min(127, x))


def test_monotone_in_x(orc):
    g = np.random.default_rng(3)
    for _ in range(20):
        M = int(g.integers(2 ** 30, 2 ** 31))
        s = int(g.integers(31, 45))
        xs = np.sort(g.integers(-2 ** 20, 2 ** 20, size=300))
        ys = [orc.requant(int(x), 0, M, s) for x in xs]
        assert all(a <= b for a, b in zip(ys, ys[1:]))


def test_bias_enters_before_multiply(orc):
    # with M = 2^30, shift = 31 the result depends on acc + bias only
    for acc, bias in [(10, 5), (-3, 2), (200, 60), (-100, -160)]:
        assert orc.requant(acc, bias, 2 ** 30, 31) == orc.requant(acc + bias, 0, 2 ** 30, 31)


def test_domain_errors(orc):
    with pytest.raises(orc.OracleDomainError):
        orc.requant(2 ** 31 - 1, 1, 2 ** 30, 31)  # acc + bias leaves int32
    with pytest.raises(orc.OracleDomainError):
        orc.requant(1, 0, 2 ** 30, 0)
    with pytest.raises(orc.OracleDomainError):
        orc.requant(1, 0, 2 ** 30, 64)
    with pytest.raises(orc.OracleDomainError):
        orc.requant(1, 0, -1, 31)
