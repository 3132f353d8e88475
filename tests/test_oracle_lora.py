"""Pins of the oracle's LoRA attachment (the adapter joins the 16-bit branch; SVDQ "feature
list": low-rank adapters integrate without re-quantizing the 4-bit residual)."""
import numpy as np

from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16
from synthetic import make_linear


def _setup(seed=0, M=48, K=256, N=96, r=16, rl=16):
    d = make_linear(2, M=M, K=K, N=N, seed=seed)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, r)
    rng = np.random.default_rng(seed + 100)
    A = round_bf16(rng.standard_normal((K, rl)) / np.sqrt(K))
    B = round_bf16(rng.standard_normal((rl, N)) * 0.1)
    return d, pw, A, B


def test_branch_gains_exactly_the_adapter_product():
    # linearity of the branch: (X^ L1') L2' = (X^ L1) L2 + X^ (lam A)(s B), checked in fp64
    d, pw, A, B = _setup()
    L1p, L2p = osq.attach_lora(pw["L1b"], pw["L2b"], pw["lam32"], A, B, scale=0.5)
    assert L1p.shape == (256, 32) and L2p.shape == (32, 96)
    Xh = osq.smooth_activations(d["X"], pw["inv_lambda"])
    base = (Xh @ pw["L1b"]) @ pw["L2b"]
    extra = (Xh @ round_bf16(pw["lam32"].astype(np.float64)[:, None] * A)) @ round_bf16(0.5 * B)
    got = (Xh @ L1p) @ L2p
    np.testing.assert_allclose(got, base + extra, rtol=0, atol=1e-9 * np.abs(base).max())


def test_adapter_acts_on_the_unsmoothed_activations():
    # with power-of-two smoothing factors every rounding above is exact, so the branch adds
    # exactly scale * X A B: the adapter sees X, not X^ (a missing or inverted lam fails here)
    d, pw, A, B = _setup(seed=1)
    K = A.shape[0]
    lam32 = np.float32(2.0) ** np.arange(-3, 5, dtype=np.float32)[np.arange(K) % 8]
    inv32 = (np.float32(1) / lam32).astype(np.float32)
    L1p, L2p = osq.attach_lora(np.zeros((K, 0)), np.zeros((0, B.shape[1])), lam32, A, B, 0.25)
    X = decode_bf16(d["X"])
    Xh = osq.smooth_activations(d["X"], inv32)
    np.testing.assert_array_equal(Xh, X * (1.0 / lam32.astype(np.float64)))  # exact scaling
    np.testing.assert_allclose((Xh @ L1p) @ L2p, 0.25 * (X @ A) @ B, rtol=1e-12,
                               atol=1e-12 * np.abs(X @ A @ B).max())


def test_residual_codes_are_untouched():
    d, pw, A, B = _setup(seed=2)
    before = osq.pack_weights(pw["R32"])
    osq.attach_lora(pw["L1b"], pw["L2b"], pw["lam32"], A, B)
    after = osq.pack_weights(pw["R32"])
    np.testing.assert_array_equal(before["wq"], after["wq"])
    np.testing.assert_array_equal(before["s_w"].view(np.uint16), after["s_w"].view(np.uint16))
    # and the attached branch stays exactly representable in bf16 (what the kernels read)
    L1p, L2p = osq.attach_lora(pw["L1b"], pw["L2b"], pw["lam32"], A, B)
    np.testing.assert_array_equal(round_bf16(L1p), L1p)
    np.testing.assert_array_equal(round_bf16(L2p), L2p)
    assert bf16_to_bits(L1p).dtype == np.uint16
