"""The activation pass on its balanced grid, against the oracle.

With long K (at least 96 groups) and between one and two 16-row blocks per CU, the pass runs
one workgroup per CU, each with an equal share of the (row block, group) units.  A share holds
at least G and at most 2 G units, so it can span three row blocks, and a row block split
between two shares gets its T as two partial sums added onto a T the call zeroes first.
Shapes (on a 256-CU device): 4608 tokens at G = 97 (shares of 109-110 units, some spanning
three row blocks), a ragged 4100 tokens (257 row blocks; 258 in the BF6 container, which is
written up to the next multiple of 32 rows), and rank 0.  Every container: codes and scales
bit-exact, T within the output tolerance, guard bands past M untouched, and the same T bits
on a second call.
"""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, round_bf16
from synthetic import make_linear
from tests.gpu_cases import dev, dev_bf16, host_u16, max_abs_rel

pytestmark = pytest.mark.gpu
TOL = 1e-2
GUARD_T, GUARD_S, GUARD_Q = -7.0, -3.0, 0x5A


def _inputs(M, K, r):
    d = make_linear(3, seed=11, M=M, K=K, N=8)
    rng = np.random.default_rng(M + K + r)
    inv = (rng.random(K) + 0.5).astype(np.float32)
    L1b = round_bf16(rng.standard_normal((K, r)) * 0.02) if r else None
    return d["X"], inv, L1b


def _run(route, X, inv, L1, M, K, r):
    G = K // 64
    xs = torch.full((M + 1, G), GUARD_S, dtype=torch.float16, device="cuda")
    T = torch.full((M + 1, max(r, 1)), GUARD_T, dtype=torch.float32, device="cuda")
    Tv = T[:M, :r] if r else None
    if route == "e3m2":
        n = B.svdq_e3m2_bytes(M, K)
        xq = torch.full((n + 64,), GUARD_Q, dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act_e3m2(X, inv, L1, r, xq[:n], xs[:M], Tv)
    elif route == "nibbles":
        xq = torch.full((M + 1, K // 2), GUARD_Q, dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act(X, inv, L1, r, xq[:M], xs[:M], Tv)
    else:
        xq = torch.full((M + 1, K), GUARD_Q, dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act_a8(X, inv, L1, r, xq[:M].view(torch.int8), xs[:M], Tv)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), host_u16(xs), T.cpu().numpy()


@pytest.mark.parametrize("M,K,r", [(4608, 6208, 16), (4100, 6144, 32), (5000, 6144, 0)])
def test_balanced_grid_matches_the_oracle(gpu_lib, M, K, r):
    Xb, inv, L1b = _inputs(M, K, r)
    ref = osq.quantize_act(Xb, inv, L1b)
    ref8 = osq.quantize_act_a8(Xb, inv, L1b)
    X, invd = dev_bf16(Xb), dev(inv)
    L1 = dev_bf16(np.ascontiguousarray(bf16_to_bits(L1b.T))) if r else None  # [r, K]
    for route in ("e3m2", "nibbles", "a8"):
        xq, xs, T = _run(route, X, invd, L1, M, K, r)
        if route == "e3m2":
            n = B.svdq_e3m2_bytes(M, K)
            np.testing.assert_array_equal(xq[:n], osq.pack_e3m2_tiled(ref["codes"]).reshape(-1))
            assert (xq[n:] == GUARD_Q).all()
        elif route == "nibbles":
            np.testing.assert_array_equal(xq[:M], ref["xq"])
            assert (xq[M] == GUARD_Q).all()
        else:
            np.testing.assert_array_equal(xq[:M].view(np.int8), ref8["xq8"])
            assert (xq[M] == GUARD_Q).all()
        want_s = np.ascontiguousarray((ref8 if route == "a8" else ref)["s_x"]).view(np.uint16)
        np.testing.assert_array_equal(xs[:M], want_s)
        assert (xs[M] == np.float16(GUARD_S).view(np.uint16)).all()
        assert (T[M] == GUARD_T).all()
        if r:
            assert max_abs_rel(T[:M].astype(np.float64), ref["T"]) <= TOL
            _, _, T2 = _run(route, X, invd, L1, M, K, r)  # two partial sums: same bits again
            np.testing.assert_array_equal(T2.view(np.uint32), T.view(np.uint32))
