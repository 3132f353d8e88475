"""Oracle of attention that reads the INT8 KV cache (the consumer of the KV quantizer).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__`` for the page short names).

VARC "INT8 KV cache quantization" stores the cache as per-channel INT8 codes with a scale and
a zero point; the memory saving becomes a runtime saving when attention reads the codes.
Reading (the page gives no attention formula): decode-time attention of nq query vectors per
head over every cached token, on the exactly dequantized cache

    K'[t, h, d] = (qk[t, h D + d] - zk[h D + d]) * sk[h D + d]      (likewise V')
    out[i, h, :] = softmax_t(sm_scale * q[i, h, :] . K'[t, h, :]) V'[t, h, :]

evaluated in fp64 (q given as bf16 bits [nq, heads, dim]).
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16


def dequantize_exact(codes, scale, zero) -> np.ndarray:
    """(q - z) * s in fp64 (no rounding), [T, C]."""
    return ((np.asarray(codes, dtype=np.float64) - np.asarray(zero, dtype=np.float64)[None, :])
            * np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :])


def attention(q_bits, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, heads: int, dim: int,
              sm_scale: float) -> np.ndarray:
    """out fp64 [nq, heads, dim]."""
    q = decode_bf16(np.asarray(q_bits, dtype=np.uint16)).reshape(-1, heads, dim)
    T = np.asarray(k_codes).shape[0]
    K = dequantize_exact(k_codes, k_scale, k_zero).reshape(T, heads, dim)
    V = dequantize_exact(v_codes, v_scale, v_zero).reshape(T, heads, dim)
    out = np.empty((q.shape[0], heads, dim), dtype=np.float64)
    for h in range(heads):
        s = sm_scale * (q[:, h, :] @ K[:, h, :].T)        # [nq, T]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, h, :]
    return out
