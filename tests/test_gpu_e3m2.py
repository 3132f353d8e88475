"""GPU parity of the BF6 (E3M2) container path against the CPU oracle, through the C ABI.

The *_e3m2 entry points carry the same INT4 codes as the nibble path in 6-bit BF6 patterns,
in the tiled container.  Bar: the container bytes equal the oracle's codes packed by the
oracle's own tiled E3M2 packer (bit-exact), scales bit-exact, the exact group partials bit-exact, T and Y within the
normwise max-abs-rel 1e-2; and the two GEMM routes agree with each other up to fp32
summation order.
"""
import functools

import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, round_bf16
from synthetic import make_linear
from tests.gpu_cases import (oracle_output, FULL, SMALL, dev, dev_bf16, device_weights, host_u16, linear_case,
                             max_abs_rel, oracle_act, with_bias)

pytestmark = pytest.mark.gpu
TOL = 1e-2
CASES = {**SMALL, **FULL}


def _case(name, bias=False):
    cid, M, K, N = CASES[name]
    return linear_case(cid, M, K, N, bias)


@functools.lru_cache(maxsize=None)
def _expected(name):
    """The oracle's codes of the case in the E3M2 container (weights, activations)."""
    case = _case(name)
    ref = oracle_act(case)
    return (osq.pack_e3m2_tiled(case[2]["codes"]).reshape(-1),
            osq.pack_e3m2_tiled(ref["codes"]).reshape(-1))


def _gpu_pack6(case):
    d, pw, packed, r = case
    K, N = pw["R32"].shape
    w = device_weights(case)
    wq6 = torch.empty(B.svdq_e3m2_bytes(N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights_e3m2(w["R32"], wq6, ws)
    return wq6, ws


def _gpu_act6(case):
    d, pw, packed, r = case
    M, K = d["X"].shape
    w = device_weights(case)
    xq6 = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(M, r, dtype=torch.float32, device="cuda") if r else None
    B.svdq_quantize_act_e3m2(dev_bf16(d["X"]), w["inv_lambda"], w["L1p"], r, xq6, xs, T)
    return xq6, xs, T


@pytest.mark.parametrize("name", list(CASES))
def test_pack_weights_e3m2_bitexact(gpu_lib, name):
    case = _case(name)
    wq6, ws = _gpu_pack6(case)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wq6.cpu().numpy(), _expected(name)[0])
    np.testing.assert_array_equal(host_u16(ws), case[2]["s_w"].view(np.uint16))


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_act_e3m2_bitexact_codes_and_lowrank(gpu_lib, name):
    case = _case(name)
    xq6, xs, T = _gpu_act6(case)
    torch.cuda.synchronize()
    ref = oracle_act(case)
    np.testing.assert_array_equal(xq6.cpu().numpy(), _expected(name)[1])
    np.testing.assert_array_equal(host_u16(xs), np.ascontiguousarray(ref["s_x"]).view(np.uint16))
    assert max_abs_rel(T.cpu().numpy().astype(np.float64), ref["T"]) <= TOL


@pytest.mark.parametrize("name,bias", with_bias(CASES))
def test_gemm_e3m2_output_within_tolerance(gpu_lib, name, bias):
    """Every row of Y against the oracle's fp64 output, in the launch configuration of the
    benchmark at the full shapes."""
    cid, M_, K_, N_ = CASES[name]
    case = _case(name, bias)
    d, pw, packed, r = case
    M = d["X"].shape[0]
    N = pw["R32"].shape[1]
    w = device_weights(case)
    wq, ws = _gpu_pack6(case)
    xq, xs, T = _gpu_act6(case)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm_e3m2(xq, xs, T, wq, ws, w["L2p"], w["bias"], r, Y)
    torch.cuda.synchronize()
    Y_ref = oracle_output(cid, M_, K_, N_, d["bias"])
    err = max_abs_rel(Y.float().cpu().numpy().astype(np.float64), Y_ref)
    assert err <= TOL, err


@pytest.mark.parametrize("cid", [1, 2])      # rank 16 and rank 32
@pytest.mark.parametrize("K", [64, 192, 320])  # one, two (ragged) and three (ragged) stages
def test_gemm_e3m2_short_k(gpu_lib, cid, K):
    # few K stages: the epilogue operands are staged from the first or a middle iteration
    case = linear_case(cid, 70, K, 100, True)
    d, pw, packed, r = case
    w = device_weights(case)
    wq6, ws = _gpu_pack6(case)
    xq6, xs, T = _gpu_act6(case)
    Y = torch.empty(70, 100, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm_e3m2(xq6, xs, T, wq6, ws, w["L2p"], w["bias"], r, Y)
    torch.cuda.synchronize()
    ref = oracle_act(case)
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                              ref["T"], pw["L2b"], d["bias"])
    assert max_abs_rel(Y.float().cpu().numpy().astype(np.float64), Y_ref) <= TOL


@pytest.mark.parametrize("name", list(CASES))
def test_partials_e3m2_bitexact(gpu_lib, name):
    """Exact int32 group partials; at the full shapes on the leading 160 x 200 and on the
    trailing 160 x 192 rows x columns (whole 32-row blocks of each container)."""
    case = _case(name)
    xq6, xs, T = _gpu_act6(case)
    wq6, ws = _gpu_pack6(case)
    d, pw = case[0], case[1]
    (M, K), N = d["X"].shape, pw["R32"].shape[1]
    G = K // 64
    ref = oracle_act(case)
    blk = G * 1536  # bytes of one 32-row block of a container
    parts = [(0, M, 0, N)]
    if name in FULL:
        assert (M - 160) % 32 == 0 and (N - 192) % 32 == 0
        parts = [(0, 160, 0, 200), (M - 160, 160, N - 192, 192)]
    for m0, mm, n0, nn in parts:
        xs6 = xq6[(m0 // 32) * blk:(m0 // 32) * blk + B.svdq_e3m2_bytes(mm, K)]
        ws6 = wq6[(n0 // 32) * blk:(n0 // 32) * blk + B.svdq_e3m2_bytes(nn, K)]
        P = torch.empty(G, mm, nn, dtype=torch.int32, device="cuda")
        B.svdq_w4a4_partials_e3m2(xs6, ws6, mm, nn, K, P)
        torch.cuda.synchronize()
        P_ref = osq.int_partials(ref["codes"][m0:m0 + mm], case[2]["codes"][n0:n0 + nn])
        np.testing.assert_array_equal(P.cpu().numpy(), P_ref)


@pytest.mark.parametrize("K", [64, 192, 320])  # G = 1, 3, 5: the last stage holds one group
def test_partials_e3m2_odd_groups_bitexact(gpu_lib, K):
    # the missing second group of the last stage is loaded from the next row block, or out of
    # range for the tensor's last row block, and never used
    case = linear_case(2, 70, K, 100)
    xq6, xs, T = _gpu_act6(case)
    wq6, ws = _gpu_pack6(case)
    P = torch.empty(K // 64, 70, 100, dtype=torch.int32, device="cuda")
    B.svdq_w4a4_partials_e3m2(xq6, wq6, 70, 100, K, P)
    torch.cuda.synchronize()
    ref = oracle_act(case)
    np.testing.assert_array_equal(P.cpu().numpy(), osq.int_partials(ref["codes"], case[2]["codes"]))


def test_e3m2_and_nibble_routes_agree(gpu_lib):
    """Same codes in both containers, and the same Y up to fp32 summation order."""
    case = _case("c3s", bias=True)
    d, pw, packed, r = case
    M, N = d["X"].shape[0], pw["R32"].shape[1]
    w = device_weights(case)
    K = d["X"].shape[1]
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(M, r, dtype=torch.float32, device="cuda")
    B.svdq_quantize_act(dev_bf16(d["X"]), w["inv_lambda"], w["L1p"], r, xq, xs, T)
    wq = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights(w["R32"], wq, ws)
    xq6, xs6, T6 = _gpu_act6(case)
    wq6, ws6 = _gpu_pack6(case)
    Y4 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Y6 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.svdq_w4a4_gemm(xq, xs, T, wq, ws, w["L2p"], w["bias"], r, Y4)
    B.svdq_w4a4_gemm_e3m2(xq6, xs6, T6, wq6, ws6, w["L2p"], w["bias"], r, Y6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(osq.unpack_e3m2_tiled(xq6.cpu().numpy(), M, K), osq.unpack_nibbles(xq.cpu().numpy()))
    np.testing.assert_array_equal(osq.unpack_e3m2_tiled(wq6.cpu().numpy(), N, K), osq.unpack_nibbles(wq.cpu().numpy()))
    assert torch.equal(xs, xs6) and torch.equal(ws, ws6) and torch.equal(T, T6)
    assert max_abs_rel(Y6.cpu().numpy().astype(np.float64), Y4.cpu().numpy().astype(np.float64)) <= 1e-5


def test_e3m2_rank0_unit_scales_reduce_to_exact_integer_gemm(gpu_lib):
    rng = np.random.default_rng(21)
    M, K, N = 200, 320, 272

    def ints(rows):
        v = rng.integers(-7, 8, (rows, K)).astype(np.float64)
        v[:, ::64] = 7.0 * rng.choice([-1.0, 1.0], (rows, K // 64))
        return v

    X, Wt = ints(M), ints(N)
    exact = X @ Wt.T
    inv = torch.ones(K, dtype=torch.float32, device="cuda")
    xq6 = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    B.svdq_quantize_act_e3m2(dev_bf16(bf16_to_bits(X)), inv, None, 0, xq6, xs, None)
    wq6 = torch.empty(B.svdq_e3m2_bytes(N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights_e3m2(dev(np.ascontiguousarray(Wt.T).astype(np.float32)), wq6, ws)
    Y32 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Y16 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm_e3m2(xq6, xs, None, wq6, ws, None, None, 0, Y32)
    B.svdq_w4a4_gemm_e3m2(xq6, xs, None, wq6, ws, None, None, 0, Y16)
    torch.cuda.synchronize()
    assert (xs.float() == 1).all() and (ws.float() == 1).all()
    np.testing.assert_array_equal(Y32.cpu().numpy().astype(np.float64), exact)
    ref16 = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(Y16.cpu().view(torch.int16), ref16.view(torch.int16))


def test_e3m2_clamped_codes_of_subnormal_scales(gpu_lib):
    """Groups with max 10 * 2^-24: the fp16 scale rounds down to 2^-24, so -max codes to the
    clamp value -8 (pattern 0x38) and +max to 7 -- the one code outside [-7, 7]."""
    rng = np.random.default_rng(22)
    M, K = 64, 256
    a = 10.0 * 2.0 ** -24
    X = round_bf16(rng.uniform(-a, a, (M, K)))
    X[:, ::64] = -a
    X[:, 1::64] = a
    bits = bf16_to_bits(X)
    inv = np.ones(K, np.float32)
    ref = osq.quantize_act(bits, inv, None)
    assert (ref["codes"] == -8).sum() >= M * K // 64 and float(ref["s_x"].max()) == 2.0 ** -24
    xq6 = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    B.svdq_quantize_act_e3m2(dev_bf16(bits), dev(inv), None, 0, xq6, xs, None)
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    xs4 = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    B.svdq_quantize_act(dev_bf16(bits), dev(inv), None, 0, xq, xs4, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq6.cpu().numpy(), osq.pack_e3m2_tiled(ref["codes"]).reshape(-1))
    np.testing.assert_array_equal(xq.cpu().numpy(), ref["xq"])


@pytest.mark.parametrize("M,K,N,r", [(1, 64, 24, 16), (17, 192, 136, 32), (129, 320, 129, 48),
                                     (7, 128, 1, 0), (300, 576, 260, 128),
                                     # more ragged tiles at G = 6, 10 and 24 groups
                                     (130, 384, 260, 32), (45, 640, 72, 16), (257, 1536, 129, 0),
                                     # G = 96 and 97: the activation pass splits K in two
                                     # (and at rank 0, with no T to combine)
                                     (37, 6144, 72, 32), (65, 6208, 40, 16), (33, 6144, 40, 0)])
def test_e3m2_ragged_shapes_with_guard_bands(gpu_lib, M, K, N, r):
    d = make_linear(3, M=M, K=K, N=N, with_bias=True)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, r)
    packed = osq.pack_weights(pw["R32"])
    ref = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
    G = K // 64
    BW, BX = B.svdq_e3m2_bytes(N, K), B.svdq_e3m2_bytes(M, K)
    GUARD = 0x5A
    wq6 = torch.full((BW + 64,), GUARD, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(G * N + 8, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights_e3m2(dev(pw["R32"]), wq6[:BW], ws[:G * N].view(G, N))
    xq6 = torch.full((BX + 64,), GUARD, dtype=torch.uint8, device="cuda")
    xs = torch.full((G * M + 8,), -3.0, dtype=torch.float16, device="cuda")
    T = torch.full((M + 1, max(r, 1)), -7.0, dtype=torch.float32, device="cuda")
    L1t = dev_bf16(bf16_to_bits(pw["L1b"].T)) if r else None
    L2t = dev_bf16(np.ascontiguousarray(bf16_to_bits(pw["L2b"]).T)) if r else None  # [N, r]
    Tv = T[:M] if r else None
    B.svdq_quantize_act_e3m2(dev_bf16(d["X"]), dev(pw["inv_lambda"]), L1t, r, xq6[:BX],
                             xs[:G * M].view(M, G), Tv)
    Y = torch.full((M + 1, N), 3.0, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm_e3m2(xq6[:BX], xs[:G * M].view(M, G), Tv, wq6[:BW], ws[:G * N].view(G, N),
                          L2t, dev_bf16(d["bias"]), r, Y[:M])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wq6[:BW].cpu().numpy(), osq.pack_e3m2_tiled(packed["codes"]).reshape(-1))
    np.testing.assert_array_equal(xq6[:BX].cpu().numpy(), osq.pack_e3m2_tiled(ref["codes"]).reshape(-1))
    assert (wq6[BW:].cpu() == GUARD).all() and (xq6[BX:].cpu() == GUARD).all()
    assert (xs[G * M:].cpu() == -3.0).all() and (ws[G * N:].cpu() == 0).all()
    assert (Y[M].cpu().float() == 3.0).all()
    if r:
        assert (T[M].cpu() == -7.0).all()
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                              ref["T"], pw["L2b"], d["bias"])
    assert max_abs_rel(Y[:M].float().cpu().numpy().astype(np.float64), Y_ref) <= TOL


def test_e3m2_fp32_output_and_determinism(gpu_lib):
    case = _case("c2s", bias=True)
    d, pw, packed, r = case
    w = device_weights(case)
    M, N = d["X"].shape[0], pw["R32"].shape[1]
    wq6, ws = _gpu_pack6(case)
    xq6, xs, T = _gpu_act6(case)
    Ya = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Yb = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.svdq_w4a4_gemm_e3m2(xq6, xs, T, wq6, ws, w["L2p"], w["bias"], r, Ya)
    B.svdq_w4a4_gemm_e3m2(xq6, xs, T, wq6, ws, w["L2p"], w["bias"], r, Yb)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb)
    ref = oracle_act(case)
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                              ref["T"], pw["L2b"], d["bias"])
    assert max_abs_rel(Ya.cpu().numpy().astype(np.float64), Y_ref) <= TOL
