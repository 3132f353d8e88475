"""Pins of the oracle's W4A8 variant: 8-bit symmetric activation codes per (token, 64-group)
(W4A8 page, sections 1 and 3.1: activations are integers from -128 to 127 and the scale is the
max magnitude over 2^(bits-1) - 1 = 127), multiplied with the same INT4 weight codes."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import svdquant as osq
from oracle.numerics import round_fp16
from synthetic import make_linear
from tests.test_oracle_quantizer import _fl32_of_fraction, _near_tie_groups, _rne_int

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def _quantize_group_exact8(v32):
    amax = max(abs(Fraction(float(t))) for t in v32)
    s16 = np.float16(_fl32_of_fraction(amax / 127))
    if float(s16) == 0.0:
        return [0] * len(v32), s16
    s = Fraction(float(s16))
    return [min(127, max(-128, _rne_int(Fraction(float(_fl32_of_fraction(Fraction(float(t)) / s))))))
            for t in v32], s16


def test_code_range_and_denominator_match_the_page():
    lo, hi = json.load(open(GOLDEN))["int8_code_range"]["value"]
    v = np.zeros(64, np.float32)
    v[0], v[1] = 63.5, -63.5          # scale exactly 0.5 (denominator 2^7 - 1 = 127)
    q, s = osq.quantize_groups(v[None], bits=8)
    assert float(s[0]) == 0.5 and q[0, :2].tolist() == [127, -127]
    # the clamp is reached only through a rounded-down subnormal scale: amax / 127 = 1.4 * 2^-24
    # rounds to 2^-24, so the quotients are +-177.8 and clamp to the page's range ends
    amax = np.float32(1.4 * 2.0 ** -24 * 127)
    v = np.zeros(64, np.float32)
    v[0], v[1] = amax, -amax
    q, s = osq.quantize_groups(v[None], bits=8)
    assert float(s[0]) == 2.0 ** -24
    assert q[0, :2].tolist() == [hi, lo] == [127, -128]


def test_hand_example_unit_scale_ties_to_even():
    v = np.zeros(64, np.float32)
    v[:7] = [127.0, 2.5, -2.5, 0.5, -100.5, 3.4999998, 55.5]
    q, s = osq.quantize_groups(v[None], bits=8)
    assert float(s[0]) == 1.0
    assert q[0, :7].tolist() == [127, 2, -2, 0, -100, 3, 56]


def test_quantizer8_matches_exact_rational_brute_force():
    rng = np.random.default_rng(15)
    groups = [rng.standard_normal(64).astype(np.float32) * np.float32(10 ** rng.uniform(-3, 3))
              for _ in range(20)]
    # near-ties at the 8-bit scale: (k + 1/2) s nudged by a few ulps
    for _ in range(20):
        amax = np.float32(rng.uniform(0.01, 50.0))
        s8 = np.float32(round_fp16(amax / np.float32(127.0)))
        k = rng.integers(-127, 127, 64)
        v = ((k + 0.5) * float(s8)).astype(np.float32)
        for i in range(64):
            for _ in range(int(rng.integers(0, 3))):
                v[i] = np.nextafter(v[i], np.float32(np.inf if rng.random() < 0.5 else -np.inf))
        v[0] = amax
        groups.append(np.clip(v, -amax, amax))
    groups += list(_near_tie_groups(rng, 4))
    groups = np.array(groups, np.float32)
    q, s = osq.quantize_groups(groups, bits=8)
    for i, g in enumerate(groups):
        codes, s16 = _quantize_group_exact8(g)
        assert float(s[i]) == float(s16), i
        assert q[i].tolist() == codes, i


def test_act_a8_codes_reconstruct_within_half_a_step_and_feed_the_integer_gemm():
    d = make_linear(2, M=40, K=256, N=48, seed=4)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, 16)
    a8 = osq.quantize_act_a8(d["X"], pw["inv_lambda"], pw["L1b"])
    a4 = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
    Xh = a8["X_hat"].astype(np.float64)
    s = np.repeat(a8["s_x"].astype(np.float64), 64, axis=1)
    assert np.all(np.abs(a8["codes"] * s - Xh) <= s / 2 * (1 + 1e-6))
    assert a8["codes"].min() >= -128 and a8["codes"].max() <= 127
    np.testing.assert_array_equal(a8["T"], a4["T"])   # same smoothing and low-rank branch
    # 8-bit activations are closer to X^ than 4-bit ones (per-group error bound s/2 vs s4/2)
    s4 = np.repeat(a4["s_x"].astype(np.float64), 64, axis=1)
    assert np.abs(a8["codes"] * s - Xh).max() < np.abs(a4["codes"] * s4 - Xh).max()
    # the integer partials with 8-bit activation codes against a pure-Python triple loop
    packed = osq.pack_weights(pw["R32"])
    P = osq.int_partials(a8["codes"][:5], packed["codes"][:7])
    np.testing.assert_array_equal(P, osq.int_partials_bruteforce(a8["codes"][:5], packed["codes"][:7]))
