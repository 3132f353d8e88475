"""Pins of the oracle's integer group GEMM and output assembly: brute force, special cases
that reduce to a plain integer GEMM or to the low-rank product alone, and shape checks that a
transposed operand would fail."""
import numpy as np

from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16
from oracle.svdquant import (int_partials, int_partials_bruteforce, linear_output, pack_weights,
                             prepare_weights, quantize_act, svdq_linear)
from synthetic import make_linear


def test_partials_match_brute_force_on_tiny_config():
    d = make_linear(1)
    pw = prepare_weights(d["X"], d["W"], 0.5, 16)
    w = pack_weights(pw["R32"])
    a = quantize_act(d["X"][:24], pw["inv_lambda"], pw["L1b"])
    cw = w["codes"][:40]
    P = int_partials(a["codes"], cw)
    Pb = int_partials_bruteforce(a["codes"].tolist(), cw.tolist())
    np.testing.assert_array_equal(P, Pb)
    assert P.shape == (256 // 64, 24, 40)


def _integer_groups(rng, rows, K):
    """Integer values in [-7, 7] where every 64-group holds a +-7 (so its scale is exactly 1)."""
    v = rng.integers(-7, 8, (rows, K)).astype(np.float64)
    v[:, ::64] = 7.0 * rng.choice([-1.0, 1.0], (rows, K // 64))
    return v


def test_rank0_unit_scale_reduces_to_integer_gemm():
    rng = np.random.default_rng(9)
    M, K, N = 37, 192, 53  # all different: a transposed operand cannot line up
    X = _integer_groups(rng, M, K)
    Wt = _integer_groups(rng, N, K)  # per output column
    W = Wt.T.copy()
    inv = np.ones(K, np.float32)
    a = quantize_act(bf16_to_bits(X), inv, None)
    w = pack_weights(W.astype(np.float32))
    np.testing.assert_array_equal(a["s_x"].astype(np.float32), 1.0)
    np.testing.assert_array_equal(w["s_w"].astype(np.float32), 1.0)
    np.testing.assert_array_equal(a["codes"], X)
    Y = linear_output(a["codes"], a["s_x"], w["codes"], w["s_w"])
    np.testing.assert_array_equal(Y, X @ W)
    # bias enters once per output column
    b = np.arange(N, dtype=np.float64) / 4.0 - 3.0
    Yb = linear_output(a["codes"], a["s_x"], w["codes"], w["s_w"], bias_bits=bf16_to_bits(b))
    np.testing.assert_array_equal(Yb, X @ W + b[None, :])


def test_zero_residual_leaves_only_the_low_rank_product():
    rng = np.random.default_rng(10)
    M, K, N, r = 20, 128, 24, 16
    L1b = decode_bf16(rng.integers(0x3C00, 0x3F80, (K, r)).astype(np.uint16))  # bf16 values
    L2b = decode_bf16(rng.integers(0x3C00, 0x3F80, (r, N)).astype(np.uint16))
    X = round_bf16(rng.standard_normal((M, K)))
    inv = np.ones(K, np.float32)
    w = pack_weights(np.zeros((K, N), np.float32))
    out = svdq_linear(bf16_to_bits(X), inv, L1b, L2b, w)
    assert not w["codes"].any()
    np.testing.assert_allclose(out["Y"], X @ L1b @ L2b, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(out["T"], X @ L1b, rtol=1e-14, atol=1e-13)


def test_group_scales_multiply_their_own_group():
    # one nonzero group per row/column pair: Y = s_x[m,g] s_w[g,n] P[g,m,n]
    K, M, N = 192, 3, 2
    X = np.zeros((M, K))
    X[0, 64:128] = 0.5
    X[0, 64] = 3.5  # amax 3.5 -> s = 0.5, codes 7 and 1
    X[1, :64] = 14.0  # s = 2, codes 7
    W = np.zeros((K, N), np.float32)
    W[64:128, 0] = 0.25  # column 0, group 1: all 0.25 -> s = 0.25/7
    W[:64, 1] = 7.0  # column 1, group 0: s = 1, codes 7
    a = quantize_act(bf16_to_bits(X), np.ones(K, np.float32), None)
    w = pack_weights(W)
    Y = linear_output(a["codes"], a["s_x"], w["codes"], w["s_w"])
    sw01 = float(w["s_w"][1, 0])
    np.testing.assert_allclose(Y[0, 0], 0.5 * sw01 * 7 * (7 + 63 * 1), rtol=1e-15)
    assert Y[1, 1] == 2.0 * 1.0 * 64 * 49
    assert Y[0, 1] == 0.0 and Y[1, 0] == 0.0 and not Y[2].any()


def test_end_to_end_error_shrinks_with_the_low_rank_branch():
    """Soft check of the pages' claim (FLUX4 2.2; VARC 'W4A4'): with outliers, SVDQuant's
    output error is below plain per-group W4A4 of the same weights."""
    d = make_linear(4, M=256, K=1024, N=256)
    X, W = decode_bf16(d["X"]), decode_bf16(d["W"])
    ref = X @ W
    pw = prepare_weights(d["X"], d["W"], 0.5, 32)
    w = pack_weights(pw["R32"])
    out = svdq_linear(d["X"], pw["inv_lambda"], pw["L1b"], pw["L2b"], w)
    e_svdq = np.linalg.norm(out["Y"] - ref)
    naive_w = pack_weights(W.astype(np.float32))
    naive = svdq_linear(d["X"], np.ones(W.shape[0], np.float32), None, None, naive_w)
    e_naive = np.linalg.norm(naive["Y"] - ref)
    assert e_svdq < 0.5 * e_naive
