"""The product path's host weight preparation (layer.prepare_host: smoothing factors, rank-r
split in bf16, fp32 residual) against the oracle's (oracle.prepare_weights), on the tiny
workload and on small shapes of the other three linear workloads.

The SVD's singular vectors are unique only up to a sign per triplet (and the two sides use
different LAPACK builds), so the factors are compared as signed pairs: rank j of (L1b, L2b)
equals the oracle's or both of its halves are the oracle's negated, which leaves L1b L2b, the
residual and its codes unchanged.  Everything else is bit-exact."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import layer
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits
from synthetic import LINEAR_CONFIGS, make_linear

CASES = [(1, None, None, None), (2, 300, 512, 384), (3, 257, 1024, 640), (4, 130, 2048, 200)]


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cid,M,K,N", CASES)
def test_prepare_host_matches_the_oracle(cid, M, K, N):
    d = make_linear(cid, M=M, K=K, N=N)
    cfg = LINEAR_CONFIGS[cid]
    pw = osq.prepare_weights(d["X"], d["W"], cfg.alpha, cfg.rank)
    hw = layer.prepare_host(_t(d["W"]), _t(d["X"]), cfg.alpha, cfg.rank)
    np.testing.assert_array_equal(hw.lam.numpy().view(np.uint32), pw["lam32"].view(np.uint32))
    np.testing.assert_array_equal(hw.inv_lambda.numpy().view(np.uint32),
                                  pw["inv_lambda"].view(np.uint32))
    L1, L2 = _u16(hw.L1b), _u16(hw.L2b)
    L1o, L2o = bf16_to_bits(pw["L1b"]), bf16_to_bits(pw["L2b"])
    for j in range(cfg.rank):
        same = np.array_equal(L1[:, j], L1o[:, j]) and np.array_equal(L2[j], L2o[j])
        flip = (np.array_equal(L1[:, j], L1o[:, j] ^ 0x8000) and
                np.array_equal(L2[j], L2o[j] ^ 0x8000))
        assert same or flip, f"rank {j}: factors differ beyond a sign"
    np.testing.assert_array_equal(hw.R32.numpy().view(np.uint32), pw["R32"].view(np.uint32))
    got, want = osq.pack_weights(hw.R32.numpy()), osq.pack_weights(pw["R32"])
    np.testing.assert_array_equal(got["wq"], want["wq"])
    np.testing.assert_array_equal(got["s_w"].view(np.uint16), want["s_w"].view(np.uint16))


def test_prepare_host_rank0_keeps_the_smoothed_weight():
    d = make_linear(1)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, 0)
    hw = layer.prepare_host(_t(d["W"]), _t(d["X"]), 0.5, 0)
    assert hw.L1b.shape == (256, 0) and hw.L2b.shape == (0, 256)
    np.testing.assert_array_equal(hw.R32.numpy().view(np.uint32), pw["R32"].view(np.uint32))
