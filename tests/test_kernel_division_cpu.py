"""The kernels' division-free roundings, checked in exact rational arithmetic on the CPU.

The activation pass forms the group scale fp16(fl32(amax / 7)) (fl32(amax / 127) in the 8-bit
variant) and the reciprocal fl32(1 / s) of that fp16 scale without a division instruction:
  * quotient by a constant d: q0 = RN(x y), r = x - d q0 (exact in one FMA), q = RN(q0 + r y),
    with y = RN(1 / d) (the correction step of Markstein's division);
  * reciprocal of an fp16 s: from a start y0 within one ulp of 1 / s (the hardware reciprocal),
    e = RN(1 - s y0), y = RN(y0 + e y0).
Both claim the correctly rounded fp32 result.  These tests evaluate every step as a fraction
rounded to fp32 by round-to-nearest-even, and compare with the correctly rounded value of the
exact quotient.  In fp32's normal range an exponent only scales every step exactly, so the
significand alone decides: the reciprocal is enumerated for all 1024 fp16 significands and
every start within two ulps; the quotient for a seeded sample of significands plus the ends of
the binade.  (No oracle or kernel code is used: this pins the arithmetic the kernels rely on.)
"""
from fractions import Fraction

import numpy as np


def _rn32(f: Fraction) -> Fraction:
    """f rounded to the nearest fp32 value (24-bit significand, ties to even), normal range."""
    if f == 0:
        return Fraction(0)
    neg = f < 0
    f = -f if neg else f
    e = f.numerator.bit_length() - f.denominator.bit_length()
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    scaled = f / Fraction(2) ** (e - 23)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = Fraction(fl) * Fraction(2) ** (e - 23)
    return -r if neg else r


def _f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def test_rn32_helper_agrees_with_numpy_on_quotients():
    rng = np.random.default_rng(3)
    for a, b in rng.integers(1, 1 << 20, size=(300, 2)):
        assert _rn32(Fraction(int(a), int(b))) == _f32(np.float32(a) / np.float32(b))


def test_reciprocal_of_every_fp16_significand_from_any_start_within_two_ulps():
    for i in range(1024):
        m = 1 + Fraction(i, 1024)
        ref = _rn32(1 / m)
        start = np.float32(float(ref))
        cands = [start]
        for direction in (np.inf, -np.inf):
            y = start
            for _ in range(2):
                y = np.nextafter(y, np.float32(direction))
                cands.append(y)
        for y0 in cands:
            y0 = Fraction(float(y0))
            e = _rn32(1 - m * y0)
            assert _rn32(y0 + e * y0) == ref, (i, y0)


def test_quotient_by_seven_and_by_127_with_the_rounded_reciprocal():
    rng = np.random.default_rng(11)
    sig = [1 << 23, (1 << 23) + 1, (1 << 24) - 1, (1 << 24) - 2]
    sig += [int(v) for v in rng.integers(1 << 23, 1 << 24, size=20000)]
    # near-ties of x / d: significands next to multiples of d (the quotient's expansion is then
    # closest to a half-ulp boundary)
    for d in (7, 127):
        base = int(rng.integers(1 << 23, (1 << 24) - 4 * d))
        base -= base % d
        sig += [base + k for k in range(-3, 4)]
    for d in (7, 127):
        y = _rn32(Fraction(1, d))
        assert y == _f32(np.float32(1.0) / np.float32(d))
        for s in sig:
            x = Fraction(s, 1 << 23)
            q0 = _rn32(x * y)
            r = x - d * q0
            assert _rn32(r) == r  # the residual is exact (one FMA)
            assert _rn32(q0 + r * y) == _rn32(x / d), (d, s)
