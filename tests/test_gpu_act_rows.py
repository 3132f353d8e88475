"""A row's activation-pass outputs do not depend on the rest of the call.

At 4608 rows the pass runs 288 workgroups of 16 rows, more than a 256-CU device holds at once.
The last 512 rows quantized in a call of their own (32 workgroups) must give the same codes,
scales and T, bit for bit: each row's outputs depend on that row alone, and T is summed in a
fixed wave order.  This covers every code container and the launch configurations of the
low-rank branch: none, rank 32 (batches of 2 groups in flight for BF6, 3 otherwise), rank 48
(batches of 6) and rank 112 (batches of 2); 8 waves per workgroup in every case.
"""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from synthetic import make_linear
from tests.gpu_cases import dev_bf16, host_u16

pytestmark = pytest.mark.gpu

M, K, TAIL = 4608, 3072, 512


def _run(route, X, inv, L1, r):
    rows = X.shape[0]
    xs = torch.empty(rows, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(rows, r, dtype=torch.float32, device="cuda") if r else None
    if route == "e3m2":
        xq = torch.empty(B.svdq_e3m2_bytes(rows, K), dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act_e3m2(X, inv, L1, r, xq, xs, T)
    elif route == "nibbles":
        xq = torch.empty(rows, K // 2, dtype=torch.uint8, device="cuda")
        B.svdq_quantize_act(X, inv, L1, r, xq, xs, T)
    else:
        xq = torch.empty(rows, K, dtype=torch.int8, device="cuda")
        B.svdq_quantize_act_a8(X, inv, L1, r, xq, xs, T)
    torch.cuda.synchronize()
    return (xq.cpu().numpy().view(np.uint8), host_u16(xs),
            T.cpu().numpy().view(np.uint32) if r else None)


@pytest.mark.parametrize("route", ["e3m2", "nibbles", "a8"])
@pytest.mark.parametrize("r", [0, 32, 48, 112])
def test_rows_alone_match_the_rows_in_a_larger_call(gpu_lib, route, r):
    g = torch.Generator().manual_seed(5)
    X = dev_bf16(make_linear(2)["X"])
    inv = (torch.rand(K, generator=g) + 0.5).cuda()
    L1 = (torch.randn(r, K, generator=g) * 0.02).to(torch.bfloat16).cuda() if r else None
    xq, xs, T = _run(route, X, inv, L1, r)
    xq_t, xs_t, T_t = _run(route, X[M - TAIL:].contiguous(), inv, L1, r)
    if route == "e3m2":  # the tail's 32-row blocks are the last TAIL / 32 of the container
        start = (M - TAIL) // 32 * (K // 64) * 1536
        np.testing.assert_array_equal(xq[start:], xq_t)
    else:
        np.testing.assert_array_equal(xq[M - TAIL:], xq_t)
    np.testing.assert_array_equal(xs[M - TAIL:], xs_t)
    if r:
        np.testing.assert_array_equal(T[M - TAIL:], T_t)
