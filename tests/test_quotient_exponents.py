"""The exponent range of the fast quotient (qar::fast_quotient, used for
block scales s >= 2^-100 with int8 and 4-bit codes, s >= 2^-90 with E4M3
codes): r = RN(1/s), y = RN(x*r), e = RN(x - y*s) (one FMA), q = RN(y + e*r)
(one FMA), emulated exactly with rationals and one binary32 rounding per
operation (tests/brute.py's rn32, gradual underflow included).

The significands are covered exhaustively on the GPU
(tests/test_gpu_quotient_exhaustive.py); the result carries over to other
exponents when scaling x and s by powers of two scales every rounded
intermediate alike.  That holds while r, y and q stay normal and the
remainder x - y*s is a multiple of 2^-149: a remainder in the subnormal
range is then exact, and one in the normal range rounds to 24 significant
bits as it does at the significands' scale (the remainder itself is not
always exact: y = RN(x*r) can be more than one spacing from x/s).  For a
quotient that decides a code (|x/s| >= 1/4 for int8 and 4-bit codes,
>= 2^-11 for E4M3) and s at or above the threshold, the remainder's quantum
2^(min(e_x - 23, e_y + e_s - 46)) is at least 2^-149.  Checked here on
sampled pairs across the scale exponents down to the thresholds, together
with q == RN(x / s) itself; smaller quotients stay in code 0's range; and
below the threshold the fast path does miss the correctly rounded quotient,
which is why the kernels divide there.
"""
from fractions import Fraction

import numpy as np
import pytest

from brute import rn32

TWO = Fraction(2)


def fast_quotient(x: Fraction, s: Fraction):
    r = rn32(1 / s)
    y = rn32(x * r)
    e = rn32(x - y * s)                    # fma(-y, s, x): one rounding of the exact value
    return rn32(e * r + y), r, y


def exponent(v: Fraction) -> int:
    """e with 2^e <= |v| < 2^(e+1) (v != 0)."""
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while TWO ** e > a:
        e -= 1
    while TWO ** (e + 1) <= a:
        e += 1
    return e


MIN_NORMAL = TWO ** -126


def premise_holds(x: Fraction, s: Fraction, r: Fraction, y: Fraction) -> bool:
    """r and y normal, and x - y*s a multiple of 2^-149."""
    if abs(r) < MIN_NORMAL or y == 0 or abs(y) < MIN_NORMAL:
        return False
    quantum = min(exponent(x) - 23, exponent(y) + exponent(s) - 46)
    return quantum >= -149


def _sig(rng):
    return Fraction(int(rng.integers(1 << 23, 1 << 24)), 1 << 23)        # a significand in [1, 2)


def _pairs(rng, exps, t_lo, t_hi, count):
    """(x, s): s a random binary32 at 2^exp, x = RN(t*s) for t log-uniform in [t_lo, t_hi]."""
    for exp in exps:
        for _ in range(count):
            s = _sig(rng) * TWO ** exp
            t = Fraction(float(np.exp(rng.uniform(np.log(t_lo), np.log(t_hi)))))
            sign = 1 if rng.integers(2) else -1
            yield sign * rn32(t * s), s


INT8_EXPS = [-100, -99, -98, -80, -40, -1, 0, 1, 50, 100, 120]
E4M3_EXPS = [-90, -89, -70, -20, 0, 30, 111]


@pytest.mark.parametrize("q_max", [127, 7])
def test_int_codes_quotients_that_decide_a_code(q_max):
    rng = np.random.default_rng(q_max)
    for x, s in _pairs(rng, INT8_EXPS, 0.25, q_max + 0.5, 150):
        q, r, y = fast_quotient(x, s)
        assert premise_holds(x, s, r, y), (x, s)
        assert q == rn32(x / s), (x, s)
    # the smallest scales themselves, with quotients just around the 0/1 decision
    for s in (TWO ** -100, (2 - TWO ** -23) * TWO ** -100, (1 + TWO ** -23) * TWO ** -100):
        for t in (Fraction(1, 4), Fraction(1, 2), Fraction(3, 4), Fraction(1, 2) + TWO ** -24,
                  Fraction(1, 2) - TWO ** -25, Fraction(-1, 2)):
            x = rn32(t * s)
            q, r, y = fast_quotient(x, s)
            assert premise_holds(x, s, r, y) and q == rn32(x / s), (t, s)


@pytest.mark.parametrize("q_max", [127, 7])
def test_int_codes_small_quotients_stay_in_code_zero(q_max):
    rng = np.random.default_rng(100 + q_max)
    for x, s in _pairs(rng, INT8_EXPS, 2.0 ** -60, 0.25, 100):
        q, _, _ = fast_quotient(x, s)
        assert abs(q) < Fraction(1, 2), (x, s)


def test_e4m3_quotients_that_decide_a_code():
    rng = np.random.default_rng(448)
    for x, s in _pairs(rng, E4M3_EXPS, 2.0 ** -11, 448.0, 150):
        q, r, y = fast_quotient(x, s)
        assert premise_holds(x, s, r, y), (x, s)
        assert q == rn32(x / s), (x, s)


def test_e4m3_small_quotients_stay_in_code_zero():
    # below 2^-10 (half the smallest subnormal E4M3 value, 2^-9) the code is +-0
    rng = np.random.default_rng(449)
    for x, s in _pairs(rng, E4M3_EXPS, 2.0 ** -60, 2.0 ** -11, 100):
        q, _, _ = fast_quotient(x, s)
        assert abs(q) < TWO ** -10, (x, s)


def test_below_the_threshold_the_fast_path_misses():
    """At scales far below 2^-100 the remainder's quantum drops under 2^-149
    and the fast path does return quotients other than the correctly
    rounded one (about 5% of code-deciding pairs at 2^-125), so the kernels
    take the IEEE division there."""
    rng = np.random.default_rng(1)
    missed = 0
    for x, s in _pairs(rng, [-125], 0.25, 127.5, 400):
        q, _, _ = fast_quotient(x, s)
        missed += q != rn32(x / s)
    assert missed > 0
