"""Oracle of the asymmetric per-channel INT8 KV-cache quantizer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__`` for the page short names).

VARC "INT8 KV cache quantization": the cache is quantized to INT8 per channel with a zero point
that is not centered, because the variance is driven by particular channels (channel CV > 1.2)
and the values are skewed (skewness about 0.85).

Readings (the page gives no formulas):
  * a channel is one (head, dim) pair; the cache [tokens, heads, dim] is viewed as x [T, C] with
    C = heads * dim, and the statistics run over every token of the call;
  * the textbook affine map with an integer zero point, over a range widened to contain 0 so
    that 0 is exactly representable:
        lo = min(0, min_t x),  hi = max(0, max_t x)           (fp32, exact on bf16 inputs)
        s  = fl32(fl32(hi - lo) / 255),  s = 1 if that is 0
        z  = clamp(rne(fl32(-lo / s)), 0, 255)                 (uint8)
        q  = clamp(rne(fl32(x / s)) + z, 0, 255)               (uint8)
        x' = bf16(fl32((q - z) * s))                           (dequantization)
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_bits, decode_bf16, round_bf16


def _as_tc(x_bits) -> np.ndarray:
    x = np.asarray(x_bits, dtype=np.uint16)
    return x.reshape(x.shape[0], -1)


def channel_params(x_bits):
    """Per-channel (scale fp32 [C], zero uint8 [C], lo fp32 [C], hi fp32 [C])."""
    x = decode_bf16(_as_tc(x_bits)).astype(np.float32)
    lo = np.minimum(np.float32(0.0), x.min(axis=0))
    hi = np.maximum(np.float32(0.0), x.max(axis=0))
    s = (hi - lo) / np.float32(255.0)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    z = np.clip(np.rint(-lo / s), 0, 255).astype(np.uint8)
    return s, z, lo, hi


def quantize(x_bits, scale, zero) -> np.ndarray:
    """uint8 codes [T, C]."""
    x = decode_bf16(_as_tc(x_bits)).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)[None, :]
    q = np.rint(x / s) + np.asarray(zero, dtype=np.float32)[None, :]
    return np.clip(q, 0, 255).astype(np.uint8)


def dequantize(q, scale, zero):
    """Returns (x' as bf16 bits [T, C], the fp32 values before the bf16 rounding)."""
    d = np.asarray(q, dtype=np.int32) - np.asarray(zero, dtype=np.int32)[None, :]
    v32 = d.astype(np.float32) * np.asarray(scale, dtype=np.float32)[None, :]
    return bf16_to_bits(round_bf16(v32.astype(np.float64))), v32


def kv_int8_quant(x_bits) -> dict:
    s, z, lo, hi = channel_params(x_bits)
    return dict(q=quantize(x_bits, s, z), scale=s, zero=z, lo=lo, hi=hi)
