"""Pins of the oracle's E3M2 (BF6) code container.

The format is fixed by the OCP Microscaling (MX) specification v1.0: 1 sign, 3 exponent
(bias 3) and 2 mantissa bits, subnormals at exponent 0, no infinities or NaNs.  Its table of
limits gives max normal 28.0, min normal 2^-2, max subnormal 0.1875 and min subnormal 0.0625;
those published values, the ordering of sign-magnitude patterns and an independent bit-level
reading of the packed stream pin the oracle's encoder, decoder and packing.
"""
import numpy as np
import pytest

from oracle.svdquant import (QMAX, QMIN, e3m2_encode_codes, e3m2_value, pack_e3m2,
                             pack_e3m2_tiled, quantize_groups, unpack_e3m2, unpack_e3m2_tiled)


def test_published_limits_of_the_format():
    assert e3m2_value(0b011111) == 28.0           # max normal
    assert e3m2_value(0b000100) == 0.25           # min normal 2^-2
    assert e3m2_value(0b000011) == 0.1875         # max subnormal
    assert e3m2_value(0b000001) == 0.0625         # min subnormal
    assert e3m2_value(0b111111) == -28.0
    assert e3m2_value(0b000000) == 0.0 and e3m2_value(0b100000) == 0.0


def test_patterns_are_sign_magnitude_ordered():
    # within one sign, a larger pattern is a strictly larger magnitude: this fixes which bits
    # are exponent and which mantissa (any other split breaks monotonicity or the limits above)
    pos = e3m2_value(np.arange(32))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(e3m2_value(np.arange(32, 64)), -pos)


def test_every_code_of_the_quantizer_round_trips_exactly():
    codes = np.arange(-8, 9)
    pat = e3m2_encode_codes(codes)
    assert np.array_equal(e3m2_value(pat), codes.astype(np.float64))
    assert len(set(pat.tolist())) == len(codes)                # injective
    assert pat[codes == 0][0] == 0                              # zero is +0
    assert QMIN >= -8 and QMAX <= 8


def test_integers_the_format_cannot_hold_are_rejected():
    # two mantissa bits: 9 = 1.001b * 2^3 and 11 = 1.011b * 2^3 need three; 29 exceeds 28
    for bad in (9, 11, -13, 29):
        with pytest.raises(ValueError):
            e3m2_encode_codes(np.array([bad]))
    assert e3m2_value(e3m2_encode_codes(np.array([10, 12, -16, 28]))).tolist() == [10, 12, -16, 28]


def test_hand_packed_stream():
    # codes 1, -1, 3, 8 -> patterns 0x0C, 0x2C, 0x12, 0x18 at stream bits 0, 6, 12, 18:
    # 0x0C | 0x2C << 6 | 0x12 << 12 | 0x18 << 18 = 0x612B0C -> bytes 0C 2B 61
    codes = np.zeros((1, 64), np.int64)
    codes[0, :4] = [1, -1, 3, 8]
    p = pack_e3m2(codes)
    assert p.shape == (1, 48)
    assert p[0, :3].tolist() == [0x0C, 0x2B, 0x61]
    assert not p[0, 3:].any()


def test_packing_against_integer_bit_extraction():
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(5, 192))
    p = pack_e3m2(codes)
    assert p.shape == (5, 144)
    pats = e3m2_encode_codes(codes)
    for r in range(5):
        stream = int.from_bytes(p[r].tobytes(), "little")
        got = [(stream >> (6 * k)) & 0x3F for k in range(192)]
        assert got == pats[r].tolist()
    assert np.array_equal(unpack_e3m2(p, 192), codes)


def test_quantizer_output_fits_the_container():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((50, 64)).astype(np.float32) * rng.uniform(1e-3, 1e3, (50, 1)).astype(np.float32)
    q, _ = quantize_groups(v)
    assert np.array_equal(unpack_e3m2(pack_e3m2(q.astype(np.int64)), 64), q)


def test_tiled_container_slot_placement_by_hand():
    # R = 33 rows (two blocks), K = 128 (two groups).  Row 32 is row 0 of block 1; its codes
    # k = 64..95 (group 1, first half) sit in block 1, group 1, slot 0; k = 96..127 in slot 32.
    R, K = 33, 128
    codes = np.zeros((R, K), np.int64)
    codes[32, 64] = 1        # -> block 1, group 1, slot 0, code 0
    codes[32, 127] = -8      # -> block 1, group 1, slot 32, code 31
    codes[5, 40] = 3         # -> block 0, group 0, slot 37 (row 5, second half), code 8
    t = pack_e3m2_tiled(codes)
    assert t.shape == (2, 2, 64, 24)
    assert t[1, 1, 0, 0] == 0x0C and not t[1, 1, 0, 1:].any()
    # code 31 occupies stream bits 186..191 = the top 6 bits of byte 23
    assert t[1, 1, 32, 23] == (0x38 << 2) & 0xFF and not t[1, 1, 32, :23].any()
    # code 8 occupies bits 48..53 = the low 6 bits of byte 6
    assert t[0, 0, 37, 6] == 0x12
    assert int(np.count_nonzero(t)) == 3
    assert not t[1, :, 1:32].any() and not t[1, :, 33:].any()   # rows past R are zero


def test_tiled_container_round_trip_and_slot_streams():
    rng = np.random.default_rng(8)
    for R, K in [(1, 64), (31, 192), (32, 64), (70, 256)]:
        codes = rng.integers(-8, 8, size=(R, K))
        t = pack_e3m2_tiled(codes)
        assert t.size == -(-R // 32) * (K // 64) * 64 * 24
        assert np.array_equal(unpack_e3m2_tiled(t, R, K), codes)
        # every slot is the plain stream of its 32 codes
        b, g, s = rng.integers(0, t.shape[0]), rng.integers(0, t.shape[1]), rng.integers(0, 64)
        row = 32 * b + s % 32
        ks = 64 * g + 32 * (s // 32)
        want = codes[row, ks:ks + 32] if row < R else np.zeros(32, np.int64)
        assert np.array_equal(t[b, g, s], pack_e3m2(want[None])[0])
