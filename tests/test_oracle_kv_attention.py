"""Pins of the oracle of attention over the INT8 KV cache: cases with closed forms (one token,
equal scores, a dominant key), token-permutation invariance, and a pure-Python brute force
that evaluates each output with a running log-sum-exp instead of a matrix softmax."""
import math

import numpy as np

from oracle import kv_attention as oka
from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16


def _case(rng, T, H=2, D=8, nq=2):
    C = H * D
    kq = rng.integers(0, 256, (T, C)).astype(np.uint8)
    vq = rng.integers(0, 256, (T, C)).astype(np.uint8)
    ks = rng.uniform(0.01, 0.05, C).astype(np.float32)
    vs = rng.uniform(0.01, 0.05, C).astype(np.float32)
    kz = rng.integers(0, 256, C).astype(np.uint8)
    vz = rng.integers(0, 256, C).astype(np.uint8)
    q = bf16_to_bits(round_bf16(rng.standard_normal((nq, H, D))))
    return q, kq, ks, kz, vq, vs, vz, H, D


def test_one_token_returns_its_value_row():
    q, kq, ks, kz, vq, vs, vz, H, D = _case(np.random.default_rng(0), T=1)
    out = oka.attention(q, kq, ks, kz, vq, vs, vz, H, D, 0.3)
    V = oka.dequantize_exact(vq, vs, vz).reshape(1, H, D)
    np.testing.assert_allclose(out, np.broadcast_to(V[0], out.shape), rtol=1e-15, atol=0)


def test_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(1)
    q, kq, ks, kz, vq, vs, vz, H, D = _case(rng, T=37)
    kq[:] = kq[0]                                  # every key the same -> uniform weights
    out = oka.attention(q, kq, ks, kz, vq, vs, vz, H, D, 0.7)
    V = oka.dequantize_exact(vq, vs, vz).reshape(37, H, D)
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=0), out.shape), rtol=1e-12)


def test_a_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    q, kq, ks, kz, vq, vs, vz, H, D = _case(rng, T=20, nq=1)
    qv = np.ones((1, H, D))
    q = bf16_to_bits(qv)
    kz[:] = 0
    kq[:] = 0
    kq[13] = 255                                   # score of token 13 exceeds the rest by ~500
    out = oka.attention(q, kq, np.full(H * D, 0.25, np.float32), kz, vq, vs, vz, H, D, 1.0)
    V = oka.dequantize_exact(vq, vs, vz).reshape(20, H, D)
    np.testing.assert_allclose(out[0], V[13], rtol=1e-12)


def test_token_order_does_not_matter():
    rng = np.random.default_rng(3)
    q, kq, ks, kz, vq, vs, vz, H, D = _case(rng, T=50)
    perm = rng.permutation(50)
    a = oka.attention(q, kq, ks, kz, vq, vs, vz, H, D, 0.4)
    b = oka.attention(q, kq[perm], ks, kz, vq[perm], vs, vz, H, D, 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-12)


def test_against_a_running_log_sum_exp_brute_force():
    rng = np.random.default_rng(4)
    q, kq, ks, kz, vq, vs, vz, H, D = _case(rng, T=9, H=2, D=4, nq=2)
    out = oka.attention(q, kq, ks, kz, vq, vs, vz, H, D, 0.5)
    qd = decode_bf16(q).reshape(2, H, D)
    for i in range(2):
        for h in range(H):
            m, l, acc = -math.inf, 0.0, [0.0] * D
            for t in range(9):
                s = 0.0
                for d in range(D):
                    c = h * D + d
                    s += qd[i, h, d] * (int(kq[t, c]) - int(kz[c])) * float(ks[c])
                s *= 0.5
                m_new = max(m, s)
                corr = math.exp(m - m_new) if m != -math.inf else 0.0
                w = math.exp(s - m_new)
                l = l * corr + w
                for d in range(D):
                    c = h * D + d
                    acc[d] = acc[d] * corr + w * (int(vq[t, c]) - int(vz[c])) * float(vs[c])
                m = m_new
            np.testing.assert_allclose(out[i, h], np.array(acc) / l, rtol=1e-12)
