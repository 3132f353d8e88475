"""Exact rounding helpers of the oracle (test infrastructure only; see ``oracle/__init__``).

* ``decode_bf16``: bf16 bit pattern -> exact float64.
* ``round_bf16``: float64 -> nearest bf16 value, ties to even, in one rounding step.
* ``bf16_to_bits``: bf16-representable float64 -> bit pattern.
* ``round_fp16``: float32 -> nearest fp16 (NumPy's conversion, which rounds to nearest even;
  pinned against a brute-force table search in the tests).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fe00000000000p+127")


def decode_bf16(bits) -> np.ndarray:
    """bf16 bits (uint16) -> float64. A bf16 value is the top half of an fp32 word."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even.

    A normal number with frexp exponent e (|x| in [2^(e-1), 2^e)) has quantum 2^(e-8) in bf16;
    below the smallest normal (2^-126, frexp exponent -125) the quantum stays 2^-133.
    Scaling by a power of two is exact in float64, and ``np.rint`` rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.rint(np.ldexp(x, 8 - e))
    y = np.ldexp(q, e - 8)
    return np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)


def bf16_to_bits(x) -> np.ndarray:
    """Bit pattern of values that are already bf16-representable (asserted)."""
    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f32.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value is not representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


def round_fp16(x32) -> np.ndarray:
    """float32 -> float16, round to nearest even (NumPy's IEEE conversion)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)
