"""GPU parity of the W4A8 variant (W4A8 page: 8-bit activations per (token, 64-group) with
scale max|x| / 127, 4-bit weights widened onto the INT8 matrix units) through the C ABI:
int8 codes and fp16 scales bit-exact, int32 group partials bit-exact, T and Y within 1e-2."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import svdquant as osq
from tests.gpu_cases import (FULL, SMALL, dev_bf16, device_weights, host_u16, linear_case,
                             max_abs_rel, with_bias)

pytestmark = pytest.mark.gpu
TOL = 1e-2
CASES = {**SMALL, "c3": FULL["c3"]}


def _case(name, bias=False):
    cid, M, K, N = CASES[name]
    return linear_case(cid, M, K, N, bias)


def _gpu(case):
    d, pw, packed, r = case
    M, K = d["X"].shape
    N = pw["R32"].shape[1]
    w = device_weights(case)
    wq = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights(w["R32"], wq, ws)
    xq8 = torch.empty(M, K, dtype=torch.int8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(M, r, dtype=torch.float32, device="cuda") if r else None
    B.svdq_quantize_act_a8(dev_bf16(d["X"]), w["inv_lambda"], w["L1p"], r, xq8, xs, T)
    return w, wq, ws, xq8, xs, T


@pytest.mark.parametrize("name", list(CASES))
def test_act_a8_codes_scales_and_lowrank(gpu_lib, name):
    case = _case(name)
    d, pw, packed, r = case
    _, _, _, xq8, xs, T = _gpu(case)
    torch.cuda.synchronize()
    ref = osq.quantize_act_a8(d["X"], pw["inv_lambda"], pw["L1b"])
    np.testing.assert_array_equal(xq8.cpu().numpy(), ref["xq8"])
    np.testing.assert_array_equal(host_u16(xs), np.ascontiguousarray(ref["s_x"]).view(np.uint16))
    assert max_abs_rel(T.cpu().numpy().astype(np.float64), ref["T"]) <= TOL


@pytest.mark.parametrize("name,bias", with_bias(CASES))
def test_w4a8_gemm_output_within_tolerance(gpu_lib, name, bias):
    case = _case(name, bias)
    d, pw, packed, r = case
    M = d["X"].shape[0]
    N = pw["R32"].shape[1]
    w, wq, ws, xq8, xs, T = _gpu(case)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a8_gemm(xq8, xs, T, wq, ws, w["L2p"], w["bias"], r, Y)
    torch.cuda.synchronize()
    ref = osq.quantize_act_a8(d["X"], pw["inv_lambda"], pw["L1b"])
    if name in FULL:
        rng = np.random.default_rng(321)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                         rng.choice(M, 32, replace=False)]))
    else:
        rows = np.arange(M)
    Y_ref = osq.linear_output(ref["codes"][rows], ref["s_x"][rows], packed["codes"],
                              packed["s_w"], ref["T"][rows] if r else None, pw["L2b"], d["bias"])
    assert max_abs_rel(Y.float().cpu().numpy()[rows].astype(np.float64), Y_ref) <= TOL


@pytest.mark.parametrize("name", list(SMALL))
def test_w4a8_partials_bitexact(gpu_lib, name):
    case = _case(name)
    d, pw, packed, r = case
    M, K = d["X"].shape
    N = pw["R32"].shape[1]
    _, wq, _, xq8, _, _ = _gpu(case)
    P = torch.empty(K // 64, M, N, dtype=torch.int32, device="cuda")
    B.svdq_w4a8_partials(xq8, wq, P)
    torch.cuda.synchronize()
    ref = osq.quantize_act_a8(d["X"], pw["inv_lambda"], pw["L1b"])
    np.testing.assert_array_equal(P.cpu().numpy(), osq.int_partials(ref["codes"], packed["codes"]))


def test_w4a8_extreme_codes_and_fp32_output(gpu_lib):
    # hand-built codes at both ends of the 8-bit and 4-bit ranges, unit scales, rank 0: the
    # fp32 output is the plain integer GEMM (every partial is exact, and so is its sum here)
    rng = np.random.default_rng(7)
    M, K, N = 130, 192, 96
    cx = rng.choice(np.array([-128, -127, -1, 0, 1, 126, 127]), size=(M, K)).astype(np.int8)
    cw = rng.choice(np.array([-8, -7, -1, 0, 1, 6, 7]), size=(N, K)).astype(np.int8)
    xq8 = torch.from_numpy(cx).cuda()
    wq = torch.from_numpy(osq.pack_nibbles(cw)).cuda()
    one = np.float16(1.0).view(np.uint16)
    xs = torch.from_numpy(np.full((M, K // 64), one, np.uint16).view(np.int16)).view(torch.float16).cuda()
    ws = torch.from_numpy(np.full((K // 64, N), one, np.uint16).view(np.int16)).view(torch.float16).cuda()
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.svdq_w4a8_gemm(xq8, xs, None, wq, ws, None, None, 0, Y)
    P = torch.empty(K // 64, M, N, dtype=torch.int32, device="cuda")
    B.svdq_w4a8_partials(xq8, wq, P)
    torch.cuda.synchronize()
    exact = cx.astype(np.int64) @ cw.astype(np.int64).T
    np.testing.assert_array_equal(Y.cpu().numpy().astype(np.int64), exact)
    np.testing.assert_array_equal(P.cpu().numpy().sum(axis=0), exact)
