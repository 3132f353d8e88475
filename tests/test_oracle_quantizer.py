"""Pins of the oracle's symmetric INT4 group quantizer and nibble packing.

The rule (W4A8 page, section 3.1, with b = 4): scale = amax / 7, q = clamp(round(v / scale),
-8, 7); the codes use the stored fp16 scale and round-half-even of the fp32 quotient.
Pins: hand-derived examples, an exact-rational brute force of IEEE fp32 division + RNE,
closed-form invariants and adversarial near-tie inputs.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.svdquant import (QMAX, QMIN, pack_nibbles, pack_weights, quantize_groups,
                             unpack_nibbles)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def test_code_range_and_denominator_match_the_page():
    pv = json.load(open(GOLDEN))
    assert [QMIN, QMAX] == pv["int4_code_range"]["value"]
    # a group whose max is 7 * 2^k gets scale exactly 2^k (denominator 7)
    v = np.zeros(64, np.float32)
    v[0] = 7.0 * 0.25
    _, s = quantize_groups(v[None])
    assert float(s[0]) == 0.25 == 7.0 * 0.25 / pv["symmetric_scale_denominator_bits4"]["value"]


def test_hand_example_unit_scale_ties_to_even():
    # amax = 7 -> fl32(7/7) = 1 -> fp16(1) = 1, so the codes are rne(v) clamped:
    # 2.5 -> 2 and -2.5 -> -2 and 0.5 -> 0 (ties to even), -3.5 -> -4, 1.5 -> 2, 6.9 -> 7
    v = np.zeros(64, np.float32)
    v[:9] = [7.0, -3.5, 2.5, -2.5, 1.5, 0.5, -0.5, 6.9, -7.0]
    q, s = quantize_groups(v[None])
    assert float(s[0]) == 1.0
    assert q[0, :9].tolist() == [7, -4, 2, -2, 2, 0, 0, 7, -7]
    assert not q[0, 9:].any()


def test_hand_example_scale_one_seventh():
    # amax = 1: fl32(1/7) = 0.142857149..., nearest fp16 is 1170 * 2^-13 = 0.142822265625.
    # 1/s = 8192/1170 = 7.0017 -> 7;  0.5/s = 3.5009 -> 4;  fl32(0.3)/s = 2.1005 -> 2;
    # -0.25/s = -1.7504 -> -2;  (s/2)/s = 0.5 exactly -> tie -> 0.
    v = np.zeros(64, np.float32)
    v[:5] = [1.0, 0.5, 0.3, -0.25, 0.0714111328125]
    q, s = quantize_groups(v[None])
    assert float(s[0]) == 1170 * 2.0 ** -13
    assert q[0, :5].tolist() == [7, 4, 2, -2, 0]


def test_zero_group_and_underflowing_scale():
    q, s = quantize_groups(np.zeros((2, 64), np.float32))
    assert not q.any() and not s.astype(np.float32).any()
    # amax / 7 below half the smallest fp16 subnormal rounds the scale to 0 -> all-zero codes
    v = np.full((1, 64), 1e-8, np.float32)
    q, s = quantize_groups(v)
    assert float(s[0]) == 0.0 and not q.any()


# ---------------------------------------------------------------- exact-rational brute force
def _fl32_of_fraction(x: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even (search around a candidate)."""
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda f: (abs(Fraction(float(f)) - x),
                                     int(np.float32(f).view(np.uint32)) & 1))
    return np.float32(best)


def _rne_int(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def _quantize_group_exact(v32):
    amax = max(abs(Fraction(float(t))) for t in v32)
    s32 = _fl32_of_fraction(amax / 7)
    s16 = np.float16(s32)  # conversion pinned separately against a brute-force table
    if float(s16) == 0.0:
        return [0] * len(v32), s16
    s = Fraction(float(s16))
    codes = []
    for t in v32:
        quot = _fl32_of_fraction(Fraction(float(t)) / s)
        codes.append(min(QMAX, max(QMIN, _rne_int(Fraction(float(quot))))))
    return codes, s16


def _near_tie_groups(rng, n_groups):
    """Groups whose elements sit at (k + 1/2) * s, nudged by a few ulps either way."""
    out = []
    for _ in range(n_groups):
        amax = np.float32(rng.uniform(0.01, 50.0))
        s = np.float32(np.float16(amax / np.float32(7.0)))
        k = rng.integers(-7, 7, 64)
        base = ((k + 0.5) * float(s)).astype(np.float32)
        nudge = rng.integers(-3, 4, 64)
        v = base.copy()
        for i in range(64):
            for _ in range(abs(int(nudge[i]))):
                v[i] = np.nextafter(v[i], np.float32(np.inf if nudge[i] > 0 else -np.inf))
        v[0] = amax
        v = np.clip(v, -amax, amax)
        out.append(v)
    return np.array(out, np.float32)


def test_quantizer_matches_exact_rational_brute_force():
    rng = np.random.default_rng(5)
    groups = [rng.standard_normal(64).astype(np.float32) * np.float32(10 ** rng.uniform(-3, 3))
              for _ in range(20)]
    groups += list(_near_tie_groups(rng, 20))
    tiny = np.full(64, 3e-7, np.float32)  # fp16-subnormal scale
    tiny[:10] = rng.uniform(-3e-7, 3e-7, 10)
    groups.append(tiny)
    groups = np.array(groups, np.float32)
    q, s = quantize_groups(groups)
    for i, g in enumerate(groups):
        codes, s16 = _quantize_group_exact(g)
        assert float(s[i]) == float(s16), i
        assert q[i].tolist() == codes, i


def test_quantizer_invariants_random():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((4000, 64)) * 10 ** rng.uniform(-2, 2, (4000, 1))).astype(np.float32)
    v[::7, 3] *= 80.0  # outliers
    q, s = quantize_groups(v)
    s32 = s.astype(np.float32)
    assert (np.abs(q) <= 7).all()  # codes never reach -8 with a normal fp16 scale
    # the element of largest magnitude codes to +-7
    i = np.argmax(np.abs(v), axis=1)
    top = q[np.arange(len(v)), i]
    assert (np.abs(top) == 7).all()
    assert (np.sign(top) == np.sign(v[np.arange(len(v)), i])).all()
    # reconstruction error at most half a step (plus the fp32 quotient rounding)
    err = np.abs(v.astype(np.float64) - q * s32[:, None].astype(np.float64))
    assert (err <= 0.5 * s32[:, None] * (1 + 2.0 ** -20)).all()


def test_pack_hand_examples_and_roundtrip():
    codes = np.array([[1, -1, -8, 7, 0, -2, 3, 5]], np.int8)
    # even k in the low nibble, two's complement: (1, -1) -> 0xF1, (-8, 7) -> 0x78,
    # (0, -2) -> 0xE0, (3, 5) -> 0x53
    assert pack_nibbles(codes).tolist() == [[0xF1, 0x78, 0xE0, 0x53]]
    rng = np.random.default_rng(7)
    c = rng.integers(-8, 8, (5, 128)).astype(np.int8)
    np.testing.assert_array_equal(unpack_nibbles(pack_nibbles(c)), c)


def test_pack_weights_groups_run_along_k_per_column():
    # R [K=128, N=3]: column n has a single large entry in group g = n % 2; the scale of
    # that (g, n) group is the only large one, which catches a transposed grouping.
    K, N = 128, 3
    R = np.full((K, N), 0.01, np.float32)
    for n in range(N):
        R[64 * (n % 2) + 5 + n, n] = 7.0
    pw = pack_weights(R)
    assert pw["wq"].shape == (N, K // 2) and pw["s_w"].shape == (K // 64, N)
    for n in range(N):
        g = n % 2
        assert float(pw["s_w"][g, n]) == 1.0
        assert pw["codes"][n, 64 * g + 5 + n] == 7
        assert float(pw["s_w"][1 - g, n]) == pytest.approx(0.01 / 7, rel=1e-3)
