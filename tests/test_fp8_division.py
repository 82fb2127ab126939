"""The fp8 cache writer divides each value of a row by the row's scale with one
correctly rounded reciprocal y = RN(1/sc) per row and three operations per
value: q = RN(x y), r = RN(x - q sc) (an FMA), result RN(q + r y) (an FMA),
its sign taken from x.  Markstein's theorem says this is RN(x / sc) when no
intermediate leaves the normal range.  This checks the claim on the CPU with
exact rational arithmetic, over random and near-tie quotients and scales from
2^-49 (the smallest the writer sends this way) to the largest a bf16 row can
give; the GPU test of the same arithmetic runs it on the device.  CPU only;
independent of the library and of the oracle."""

import math
import random
from fractions import Fraction

import numpy as np

EMIN, P = -126, 24                      # fp32: smallest normal exponent, precision


def rn32(v: Fraction) -> Fraction:
    """v rounded to the nearest fp32 value (ties to even), subnormals
    included; no overflow occurs here."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, EMIN) - (P - 1)                       # exponent of the last kept bit
    m = a / Fraction(2) ** q
    lo = math.floor(m)
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return s * lo * Fraction(2) ** q


def f32(x: float) -> Fraction:
    return Fraction(float(np.float32(x)))


def writer_div(x: Fraction, sc: Fraction) -> Fraction:
    y = rn32(1 / sc)
    q = rn32(x * y)
    r = rn32(x - q * sc)
    out = rn32(q + r * y)
    return out                                       # (x == 0 is not sampled; the sign rule covers it)


def random_f32(rng: random.Random, lo_exp: int, hi_exp: int) -> Fraction:
    """A random fp32 value with exponent in [lo_exp, hi_exp] and a random
    significand."""
    e = rng.randint(lo_exp, hi_exp)
    m = rng.randrange(1 << 23, 1 << 24)
    return Fraction(m) * Fraction(2) ** (e - 23)


def test_writer_division_is_correctly_rounded():
    rng = random.Random(20261202)
    cases = 0
    for i in range(6000):
        # Scale: a bf16 row maximum / 448 spans 2^-49 .. 2^119.
        sc = rn32(random_f32(rng, -49, 118))
        mode = i % 3
        if mode == 0:                                # any quotient magnitude up to 448
            u = random_f32(rng, -12, 8)
            x = rn32(u * sc)
        elif mode == 1:                              # quotient near an fp32 tie
            q = random_f32(rng, -11, 8)
            e = math.floor(math.log2(float(q)))
            half = Fraction(2) ** (e - 24)
            x = rn32((q + half) * sc)
        else:                                        # x = the row maximum itself, quotient near 448
            x = rn32(Fraction(448) * sc * (1 + Fraction(rng.randint(-8, 8), 1 << 24)))
        if x == 0:
            continue
        if rng.random() < 0.5:
            x = -x
        want = rn32(x / sc)
        got = writer_div(x, sc)
        assert got == want, (float(x), float(sc), float(got), float(want))
        cases += 1
    assert cases > 5000


def test_the_sign_rule_is_needed_for_negative_zero():
    """Without copying x's sign, x = -0 would give +0 (code 0x00 instead of
    0x80): q = -0, r = +0 + -0 = +0, q + r y = -0 + +0 = +0."""
    sc = f32(0.75)
    y = rn32(1 / sc)
    q = -0.0 * float(y)
    r = (-q) * float(sc) + -0.0                      # exact: no rounding happens
    out = (r * float(y)) + q
    assert math.copysign(1.0, out) == 1.0
