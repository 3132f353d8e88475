"""Pins of the oracle's rounding helpers against brute-force table searches and a library
conversion (not against their own formulas)."""
import numpy as np
import pytest
import torch

from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16, round_fp16

pytestmark = pytest.mark.filterwarnings("ignore:invalid value encountered in cast")


def _finite_table(kind):
    bits = np.arange(65536, dtype=np.uint32)
    if kind == "bf16":
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        mant_bits = bits & 0x7F
    else:
        vals = bits.astype(np.uint16).view(np.float16).astype(np.float64)
        mant_bits = bits & 0x3FF
    ok = np.isfinite(vals)
    vals, mant_bits = vals[ok], mant_bits[ok]
    order = np.argsort(vals, kind="stable")
    vals, mant_bits = vals[order], mant_bits[order]
    # +0 and -0 both appear; keep one
    keep = np.concatenate([[True], np.diff(vals) != 0])
    return vals[keep], mant_bits[keep]


def _nearest_even(table, mant, x):
    """Brute force: nearest table value, ties to the one with an even last mantissa bit."""
    idx = np.searchsorted(table, x)
    idx = np.clip(idx, 1, len(table) - 1)
    lo, hi = table[idx - 1], table[idx]
    dlo, dhi = x - lo, hi - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (mant[idx] % 2 == 0))
    return np.where(pick_hi, hi, lo)


def _samples(rng, lo_exp, hi_exp, n):
    mag = 2.0 ** rng.uniform(lo_exp, hi_exp, n)
    return mag * rng.choice([-1.0, 1.0], n)


def test_round_bf16_matches_brute_force_nearest_even():
    rng = np.random.default_rng(1)
    table, mant = _finite_table("bf16")
    x = np.concatenate([_samples(rng, -130, 120, 20000),
                        # exact midpoints between neighbouring bf16 values: ties
                        0.5 * (table[1000:1400] + table[1001:1401]),
                        0.5 * (table[40000:40300] + table[40001:40301])])
    x = x[np.abs(x) < table[-1]]
    np.testing.assert_array_equal(round_bf16(x), _nearest_even(table, mant, x))


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(2)
    x32 = _samples(rng, -60, 60, 50000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x32.astype(np.float64)), ref)


def test_bf16_bits_roundtrip_and_decode():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 65536, 10000, dtype=np.uint32).astype(np.uint16)
    vals = decode_bf16(bits)
    ok = np.isfinite(vals)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals[ok], ref[ok])
    np.testing.assert_array_equal(bf16_to_bits(vals[ok]), bits[ok])
    with pytest.raises(ValueError):
        bf16_to_bits(np.array([1.0 + 2.0 ** -10]))


def test_round_fp16_matches_brute_force_nearest_even():
    rng = np.random.default_rng(4)
    table, mant = _finite_table("fp16")
    x = np.concatenate([_samples(rng, -26, 15.9, 30000),
                        0.5 * (table[100:600] + table[101:601]),        # subnormal ties
                        0.5 * (table[30000:30500] + table[30001:30501])])
    x32 = x.astype(np.float32)
    x32 = x32[np.abs(x32) < 65504]
    got = round_fp16(x32).astype(np.float64)
    np.testing.assert_array_equal(got, _nearest_even(table, mant, x32.astype(np.float64)))
