"""Pins of the oracle's asymmetric per-channel INT8 KV quantizer: hand-derived examples,
an exact-rational brute force, round-trip bounds and the page's asymmetric-vs-symmetric claim."""
from fractions import Fraction

import numpy as np

from oracle.kv_int8 import channel_params, dequantize, kv_int8_quant, quantize
from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16
from synthetic import make_kv


def _bits(a):
    return bf16_to_bits(np.asarray(a, np.float64))


def test_hand_examples():
    # tokens x channels; channel c holds column c
    x = np.array([[-1.0, 0.5, -2.0, 0.0],
                  [0.0, 0.25, -0.5, 0.0],
                  [3.0, 2.0, 0.0, 0.0]])
    r = kv_int8_quant(_bits(x))
    # ch0: lo=-1, hi=3, s=fl32(4/255); -lo/s = 63.749996 -> z=64;
    #      -1/s -> -64 + 64 = 0;  0 -> 64;  3/s = 191.24998 -> 191 + 64 = 255
    # ch1: lo=0 (widened), hi=2, s=fl32(2/255), z=0; 0.5/s=63.749996 -> 64; 0.25/s -> 32;
    #      2/s = 254.99998 -> 255
    # ch2: lo=-2, hi=0, z = rne(254.99998) = 255; -2 -> 0; -0.5 -> -64+255 = 191; 0 -> 255
    # ch3: constant zero -> range 0 -> s = 1, z = 0, codes 0
    assert r["zero"].tolist() == [64, 0, 255, 0]
    assert r["scale"][3] == 1.0
    assert r["scale"][0] == np.float32(4.0) / np.float32(255.0)
    assert r["q"].T.tolist() == [[0, 64, 255], [64, 32, 255], [0, 191, 255], [0, 0, 0]]


def _fl32(x: Fraction):
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return np.float32(min(cands, key=lambda f: (abs(Fraction(float(f)) - x),
                                                int(np.float32(f).view(np.uint32)) & 1)))


def _rne(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    return fl + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else fl


def test_matches_exact_rational_brute_force():
    d = make_kv(seed=3, tokens=48, heads=2, dim=8)
    xb = d["K"].reshape(48, 16)
    r = kv_int8_quant(xb)
    x = decode_bf16(xb)
    for c in range(16):
        col = [Fraction(float(v)) for v in x[:, c]]
        lo, hi = min(Fraction(0), min(col)), max(Fraction(0), max(col))
        s = _fl32(Fraction(float(_fl32(hi - lo))) / 255)
        s = np.float32(1.0) if s == 0 else s
        S = Fraction(float(s))
        z = min(255, max(0, _rne(Fraction(float(_fl32(-lo / S))))))
        assert r["scale"][c] == s and r["zero"][c] == z
        for t in range(48):
            q = _rne(Fraction(float(_fl32(col[t] / S)))) + z
            assert r["q"][t, c] == min(255, max(0, q)), (t, c)


def test_roundtrip_bounds_and_endpoints():
    d = make_kv(seed=1, tokens=512, heads=4, dim=16)
    xb = d["V"].reshape(512, 64)
    r = kv_int8_quant(xb)
    x = decode_bf16(xb)
    bits, v32 = dequantize(r["q"], r["scale"], r["zero"])
    s = r["scale"].astype(np.float64)
    err = np.abs(v32.astype(np.float64) - x)
    assert (err <= s[None, :] * (0.5 + 2.0 ** -14)).all()
    # the range endpoints: lo codes to exactly 0 (rne is odd-symmetric), hi to 254 or 255
    lo_idx, hi_idx = np.argmin(x, 0), np.argmax(x, 0)
    cols = np.arange(x.shape[1])
    has_neg = x[lo_idx, cols] < 0
    assert (r["q"][lo_idx, cols][has_neg] == 0).all()
    assert (r["q"][hi_idx, cols] >= 254).all()
    # dequantized values are the bf16 rounding of the fp32 products
    assert np.abs(decode_bf16(bits) - v32).max() <= np.abs(v32).max() * 2.0 ** -8


def test_statistics_run_over_tokens_per_channel():
    # channels with very different ranges: a transposed reduction would mix them
    T, C = 64, 8
    x = round_bf16(np.outer(np.linspace(-1, 1, T), 2.0 ** np.arange(C)))
    s, z, lo, hi = channel_params(_bits(x))
    np.testing.assert_array_equal(hi, np.float32(2.0 ** np.arange(C)))
    np.testing.assert_array_equal(lo, -np.float32(2.0 ** np.arange(C)))
    # power-of-two channel ranges give the same zero point everywhere (about 255/2)
    assert len(set(z.tolist())) == 1 and z[0] in (127, 128)
    np.testing.assert_array_equal(s, s[0] * np.float32(2.0 ** np.arange(C)))


def test_asymmetric_beats_symmetric_on_skewed_cache():
    """Soft check of VARC 'INT8 KV cache quantization': on skewed data the asymmetric
    per-channel map loses less than a symmetric per-channel one."""
    d = make_kv(seed=0, tokens=2048, heads=4, dim=32)
    xb = d["K"].reshape(2048, 128)
    x = decode_bf16(xb)
    r = kv_int8_quant(xb)
    _, v32 = dequantize(r["q"], r["scale"], r["zero"])
    mse_asym = np.mean((v32 - x) ** 2)
    ss = np.abs(x).max(0) / 127.0
    mse_sym = np.mean((np.clip(np.rint(x / ss), -127, 127) * ss - x) ** 2)
    assert mse_asym < mse_sym


def test_quantize_uses_given_params():
    x = _bits([[1.0, -1.0], [0.5, 2.0]])
    q = quantize(x, np.float32([0.5, 0.25]), np.uint8([10, 100]))
    assert q.tolist() == [[12, 96], [11, 108]]
