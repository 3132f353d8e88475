"""Group scales at exact fp16 ties (activation pass, all three code containers).

The scale is fp16(fl32(amax / 7)) (amax / 127 for 8-bit codes), and fp16 rounds ties to even.
These inputs make amax = d * m for m the midpoint between two adjacent fp16 values, so the fp32
quotient is exactly that midpoint (d m has at most 19 significant bits: exact in fp32, and the
correction-step quotient is exact) and the conversion must pick the even neighbour.  On this
path the compiler once fused the quotient's last FMA with the fp16 conversion
(v_fma_mixlo_f16), whose result differed from the separate conversion on scales of this kind;
the kernels keep the two apart.  Each group's maximum comes from one channel whose x is a
power of two and whose inv_lambda is the target, so x^ = x * inv_lambda hits it exactly.
"""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, round_bf16
from tests.gpu_cases import dev, dev_bf16, host_u16

pytestmark = pytest.mark.gpu


def _tie_targets(d: int, n: int, seed: int) -> np.ndarray:
    """fp32 values t = d * m, m the midpoint of two adjacent fp16 values in [2^-6, 2^7)."""
    rng = np.random.default_rng(seed)
    h = rng.integers(0x2400, 0x5800, size=n).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    t = ((lo + hi) / 2 * d).astype(np.float32)
    assert np.all(t.astype(np.float64) == (lo + hi) / 2 * d)  # exact
    return t


def _inputs(d: int, M: int, G: int, seed: int):
    K = 64 * G
    t = _tie_targets(d, G, seed)
    rng = np.random.default_rng(seed + 1)
    inv = np.ones(K, np.float32)
    inv[::64] = t
    X = np.empty((M, K))
    scale = (2.0 ** (np.arange(M) % 8 - 4))[:, None]  # per-row power of two: exact scaling
    X[:] = rng.uniform(-0.9, 0.9, (M, K)) * np.repeat(t.astype(np.float64), 64)[None, :] * scale
    X[:, ::64] = scale  # x^ = scale * t exactly: the group's maximum
    bits = bf16_to_bits(round_bf16(X))
    # every other channel's |x^| stays below the maximum (bf16 rounding of 0.9 t is < t)
    return bits, inv, t


@pytest.mark.parametrize("route", ["nibbles", "e3m2", "a8"])
def test_scales_at_fp16_ties_of_the_fp32_quotient(gpu_lib, route):
    d = 127 if route == "a8" else 7
    M, G = 32, 128
    bits, inv, t = _inputs(d, M, G, seed=5 + d)
    # every group's fp32 quotient is an fp16 tie, and half of them round down to the even side
    q = (t / np.float32(d)).astype(np.float32)
    assert np.all(q.astype(np.float64) == t.astype(np.float64) / d)
    even = q.astype(np.float16).view(np.uint16)
    assert np.all(even % 2 == 0) and np.all(q.astype(np.float16).astype(np.float64) != q)
    K = 64 * G
    ref = osq.quantize_act_a8(bits, inv, None) if route == "a8" else osq.quantize_act(bits, inv, None)
    X, invd = dev_bf16(bits), dev(inv)
    xs = torch.empty(M, G, dtype=torch.float16, device="cuda")
    if route == "nibbles":
        xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act(X, invd, None, 0, xq, xs, None)
        want = ref["xq"]
    elif route == "e3m2":
        xq = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act_e3m2(X, invd, None, 0, xq, xs, None)
        want = osq.pack_e3m2_tiled(ref["codes"]).reshape(-1)
    else:
        xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        B.svdq_quantize_act_a8(X, invd, None, 0, xq, xs, None)
        want = ref["xq8"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(xs), np.asarray(ref["s_x"]).view(np.uint16))
    np.testing.assert_array_equal(xq.cpu().numpy().reshape(-1), np.asarray(want).reshape(-1))
