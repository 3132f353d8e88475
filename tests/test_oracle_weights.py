"""Pins of the oracle's weight preparation: smoothing factors (closed forms, the smoothing
identity) and the low-rank split (Eckart-Young-Mirsky, reconstruction, special cases)."""
import numpy as np
import pytest

from oracle.numerics import round_bf16
from oracle.svdquant import low_rank_split, prepare_weights, smoothing_factors
from synthetic import make_linear


def test_smoothing_closed_form():
    # a_k = max_m |X_mk| = [4, 9, 0, 1, 2];  w_k = max_n |W_kn| = [1, 4, 2, 0, 8]
    X = np.array([[4.0, -9.0, 0.0, 1.0, 2.0], [-1.0, 3.0, 0.0, -0.5, 0.0]])
    W = np.array([[1.0, -0.5], [4.0, 2.0], [0.0, -2.0], [0.0, 0.0], [-8.0, 1.0]])
    lam, inv = smoothing_factors(X, W, 0.5)
    # sqrt(a/w) where both are nonzero; 1 where either is zero
    np.testing.assert_array_equal(lam, np.float32([2.0, 1.5, 1.0, 1.0, 0.5]))
    np.testing.assert_array_equal(inv, np.float32([0.5, 1.0 / np.float32(1.5), 1.0, 1.0, 2.0]))
    lam1, _ = smoothing_factors(X, W, 1.0)  # alpha = 1: lam = a
    np.testing.assert_array_equal(lam1, np.float32([4.0, 9.0, 1.0, 1.0, 2.0]))
    lam0, _ = smoothing_factors(X, W, 0.0)  # alpha = 0: lam = 1 / w
    np.testing.assert_array_equal(lam0, np.float32([1.0, 0.25, 1.0, 1.0, 0.125]))


def test_smoothing_identity_and_outlier_migration():
    d = make_linear(2, M=256, K=512, N=384)
    from oracle.numerics import decode_bf16
    X, W = decode_bf16(d["X"]), decode_bf16(d["W"])
    lam, inv = smoothing_factors(X, W, 0.5)
    Xh = X * inv.astype(np.float64)[None, :]
    Wh = lam.astype(np.float64)[:, None] * W
    ref = X @ W
    assert np.abs(Xh @ Wh - ref).max() <= 1e-6 * np.abs(ref).max()
    # the outlier channels' activation ranges shrink toward the others'
    ch = d["outlier_channels"]
    before = np.abs(X).max(0)
    after = np.abs(Xh).max(0)
    assert (before[ch].mean() / np.median(before)) > 5 * (after[ch].mean() / np.median(after))


@pytest.mark.parametrize("rank", [0, 1, 8, 32])
def test_eckart_young_mirsky(rank):
    rng = np.random.default_rng(8)
    Wh = rng.standard_normal((96, 160)) + 5.0 * np.outer(rng.standard_normal(96), rng.standard_normal(160))
    sp = low_rank_split(Wh, rank)
    sig = np.linalg.svd(Wh, compute_uv=False)
    E = Wh - sp["L1"] @ sp["L2"]  # with the exact (fp64) factors
    assert np.linalg.norm(E, 2) == pytest.approx(sig[rank], rel=1e-10)
    assert np.linalg.norm(E, "fro") ** 2 == pytest.approx(np.sum(sig[rank:] ** 2), rel=1e-10)
    # with the bf16 factors the residual stays within sigma_{r+1} + the rounding perturbation
    pert = np.linalg.norm(sp["L1"] @ sp["L2"] - sp["L1b"] @ sp["L2b"], 2)
    assert np.linalg.norm(sp["R"], 2) <= sig[rank] + pert + 1e-9
    # reconstruction: L1b L2b + R is W^ (fp64), and R32 is R rounded to fp32
    np.testing.assert_allclose(sp["L1b"] @ sp["L2b"] + sp["R"], Wh, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(sp["R32"], sp["R"].astype(np.float32))
    np.testing.assert_array_equal(sp["L1b"], round_bf16(sp["L1"]))


def test_exact_low_rank_weight_leaves_zero_residual():
    # W = e_0 e_3^T has one singular value 1 with unit singular vectors, which bf16 holds
    # exactly; LAPACK leaves only ~1e-16 noise in the other entries of the factors
    W = np.zeros((64, 32))
    W[0, 3] = 1.0
    sp = low_rank_split(W, 1)
    assert np.abs(sp["R"]).max() < 1e-15
    assert abs(sp["L1b"][0, 0] * sp["L2b"][0, 3]) == 1.0


def test_rank_spike_is_absorbed_on_attention_weights():
    d = make_linear(2, M=128, K=512, N=512)
    pw = prepare_weights(d["X"], d["W"], 0.5, 32)
    S = pw["S"]
    # the rank-8 spike of spectral norm 10 is in the top of the spectrum and the residual's
    # spectral norm is sigma_33 (plus the bf16 rounding of the factors)
    assert np.linalg.norm(pw["R"], 2) <= S[32] * 1.05
    assert np.linalg.norm(pw["R"], 2) < 0.5 * S[0]
