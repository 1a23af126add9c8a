"""The KIVI prefill kernel forms each code's quotient fl32(x / s) as q0 = fl32(x r), e = x - q0 s,
q = fl32(q0 + e r) with r the hardware reciprocal of s (accurate to 1 ulp), instead of a correctly
rounded division.  For fp16 x and s that is exactly the correctly rounded quotient the quantizer is
defined with (KIVI page, "definitions"); this checks it in exact rational arithmetic for every r within
1 ulp of 1/s, on random fp16 pairs and on the extremes of the fp16 range."""

import random
from fractions import Fraction as F

import numpy as np


def rn32(v: F) -> F:
    """v rounded to the nearest binary32 value, ties to even (the values here stay in the normal range)."""
    if v == 0:
        return F(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** (max(e, -126) - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > F(1, 2) or (rem == F(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f16(bits: int) -> F:
    return F(float(np.frombuffer(np.uint16(bits).tobytes(), np.float16)[0]))


def quotient_ok(x: F, s: F) -> bool:
    want = rn32(x / s)
    r0 = rn32(1 / s)
    e0 = r0.numerator.bit_length() - r0.denominator.bit_length()
    ulp = F(2) ** (e0 - 24)
    for r in (r0 - ulp, r0, r0 + ulp):
        q0 = rn32(x * r)
        e = x - q0 * s
        if rn32(e) != e:                            # the residual must be exact in one FMA
            return False
        if rn32(q0 + e * r) != want:
            return False
    return True


def test_newton_quotient_is_correctly_rounded():
    rng = random.Random(7)
    finite = list(range(0x0001, 0x7c00))            # positive finite fp16 bit patterns
    cases = [(f16(rng.choice(finite)) * rng.choice((1, -1)), f16(rng.choice(finite))) for _ in range(1500)]
    ext = [f16(0x0001), f16(0x0002), f16(0x03ff), f16(0x0400), f16(0x3c00), f16(0x3e00), f16(0x7bff)]
    cases += [(x * sg, s) for x in ext for s in ext for sg in (1, -1)]
    cases += [(F(0), f16(0x3555))]
    bad = [(float(x), float(s)) for x, s in cases if not quotient_ok(x, s)]
    assert not bad, bad[:5]
