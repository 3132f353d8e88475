"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar: codes, scales, zero points and int32 partials bit-exact; T and Y within the normwise
max-abs-rel 1e-2 of the method's output tolerance.  Small cases span several 128x128 tiles
with ragged tails; the full workload shapes run in the benchmark's launch configuration and
compare sampled output rows.
"""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import kv_int8 as okv
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, round_bf16
from synthetic import make_linear
from tests.gpu_cases import (oracle_output, FULL, SMALL, dev, dev_bf16, device_weights, host_u16, kv_case,
                             linear_case, max_abs_rel, oracle_act, with_bias)

pytestmark = pytest.mark.gpu
TOL = 1e-2
CASES = {**SMALL, **FULL}


def _case(name, bias=False):
    cid, M, K, N = CASES[name]
    return linear_case(cid, M, K, N, bias)


def _gpu_pack(case):
    d, pw, packed, r = case
    K, N = pw["R32"].shape
    w = device_weights(case)
    wq = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights(w["R32"], wq, ws)
    return wq, ws


def _gpu_act(case):
    d, pw, packed, r = case
    M, K = d["X"].shape
    w = device_weights(case)
    X = dev_bf16(d["X"])
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(M, r, dtype=torch.float32, device="cuda") if r else None
    B.svdq_quantize_act(X, w["inv_lambda"], w["L1p"], r, xq, xs, T)
    return xq, xs, T


@pytest.mark.parametrize("name", list(CASES))
def test_pack_weights_bitexact(gpu_lib, name):
    case = _case(name)
    wq, ws = _gpu_pack(case)
    torch.cuda.synchronize()
    packed = case[2]
    np.testing.assert_array_equal(wq.cpu().numpy(), packed["wq"])
    np.testing.assert_array_equal(host_u16(ws), packed["s_w"].view(np.uint16))


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_act_bitexact_codes_and_lowrank(gpu_lib, name):
    case = _case(name)
    xq, xs, T = _gpu_act(case)
    torch.cuda.synchronize()
    ref = oracle_act(case)
    np.testing.assert_array_equal(xq.cpu().numpy(), ref["xq"])
    np.testing.assert_array_equal(host_u16(xs), np.ascontiguousarray(ref["s_x"]).view(np.uint16))
    err = max_abs_rel(T.cpu().numpy().astype(np.float64), ref["T"])
    assert err <= TOL, err


def test_quantize_act_long_k_both_containers(gpu_lib):
    # K = 24576: the smoothing factors no longer fit the activation kernel's LDS budget beside
    # the rank-32 reduction area, so it reads them from global memory instead.  Both code
    # containers, codes and scales bit-exact, T within tolerance.
    case = linear_case(4, 40, 24576, 64)
    d, pw, packed, r = case
    M, K = d["X"].shape
    w = device_weights(case)
    X = dev_bf16(d["X"])
    ref = oracle_act(case)
    xq, xs, T = _gpu_act(case)
    xq6 = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
    xs6 = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T6 = torch.empty(M, r, dtype=torch.float32, device="cuda")
    B.svdq_quantize_act_e3m2(X, w["inv_lambda"], w["L1p"], r, xq6, xs6, T6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), ref["xq"])
    np.testing.assert_array_equal(xq6.cpu().numpy(), osq.pack_e3m2_tiled(ref["codes"]).reshape(-1))
    want_s = np.ascontiguousarray(ref["s_x"]).view(np.uint16)
    np.testing.assert_array_equal(host_u16(xs), want_s)
    np.testing.assert_array_equal(host_u16(xs6), want_s)
    assert max_abs_rel(T.cpu().numpy().astype(np.float64), ref["T"]) <= TOL
    assert max_abs_rel(T6.cpu().numpy().astype(np.float64), ref["T"]) <= TOL


@pytest.mark.parametrize("name,bias", with_bias(CASES))
def test_gemm_output_within_tolerance(gpu_lib, name, bias):
    """Every row of Y against the oracle's fp64 output, in the launch configuration of the
    benchmark at the full shapes."""
    cid, M_, K_, N_ = CASES[name]
    case = _case(name, bias)
    d, pw, packed, r = case
    M = d["X"].shape[0]
    N = pw["R32"].shape[1]
    w = device_weights(case)
    wq, ws = _gpu_pack(case)
    xq, xs, T = _gpu_act(case)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm(xq, xs, T, wq, ws, w["L2p"], w["bias"], r, Y)
    torch.cuda.synchronize()
    Y_ref = oracle_output(cid, M_, K_, N_, d["bias"])
    err = max_abs_rel(Y.float().cpu().numpy().astype(np.float64), Y_ref)
    assert err <= TOL, err


@pytest.mark.parametrize("name", list(CASES))
def test_partials_bitexact(gpu_lib, name):
    """Exact int32 group partials; at the full shapes (whose G M N partials do not fit in
    memory) on the leading and on the trailing 160 rows x 200 columns of the problem."""
    case = _case(name)
    d, pw, packed, r = case
    xq, xs, T = _gpu_act(case)
    wq, ws = _gpu_pack(case)
    ref = oracle_act(case)
    M, N = xq.shape[0], wq.shape[0]
    slices = [(slice(0, M), slice(0, N))]
    if name in FULL:
        slices = [(slice(0, 160), slice(0, 200)), (slice(M - 160, M), slice(N - 200, N))]
    for rs, cs in slices:
        xs_, ws_ = xq[rs].contiguous(), wq[cs].contiguous()
        G = xs_.shape[1] * 2 // 64
        P = torch.empty(G, xs_.shape[0], ws_.shape[0], dtype=torch.int32, device="cuda")
        B.svdq_w4a4_partials(xs_, ws_, P)
        torch.cuda.synchronize()
        P_ref = osq.int_partials(ref["codes"][rs], packed["codes"][cs])
        np.testing.assert_array_equal(P.cpu().numpy(), P_ref)


def test_rank0_unit_scales_reduce_to_exact_integer_gemm(gpu_lib):
    """Integer inputs in [-7, 7] with a +-7 in every group: scales are 1 and codes equal the
    inputs, so Y is the plain integer GEMM, exact in fp32 and correctly rounded in bf16."""
    rng = np.random.default_rng(11)
    M, K, N = 200, 320, 272

    def ints(rows):
        v = rng.integers(-7, 8, (rows, K)).astype(np.float64)
        v[:, ::64] = 7.0 * rng.choice([-1.0, 1.0], (rows, K // 64))
        return v

    X, Wt = ints(M), ints(N)
    exact = X @ Wt.T
    Xd = dev_bf16(bf16_to_bits(X))
    inv = torch.ones(K, dtype=torch.float32, device="cuda")
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    B.svdq_quantize_act(Xd, inv, None, 0, xq, xs, None)
    wq = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights(dev(np.ascontiguousarray(Wt.T).astype(np.float32)), wq, ws)
    Y32 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Y16 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm(xq, xs, None, wq, ws, None, None, 0, Y32)
    B.svdq_w4a4_gemm(xq, xs, None, wq, ws, None, None, 0, Y16)
    torch.cuda.synchronize()
    assert (xs.float() == 1).all() and (ws.float() == 1).all()
    np.testing.assert_array_equal(Y32.cpu().numpy().astype(np.float64), exact)
    ref16 = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(Y16.cpu().view(torch.int16), ref16.view(torch.int16))


def test_exact_ties_round_half_to_even(gpu_lib):
    """Values at exactly (k + 1/2) * s (and one bf16 ulp either side) for power-of-two scales."""
    rng = np.random.default_rng(12)
    M, K = 48, 256
    e = rng.integers(-6, 6, (M, K // 64)).astype(np.float64)
    s = np.repeat(2.0 ** e, 64, axis=1)
    k = rng.integers(-7, 7, (M, K)).astype(np.float64)
    X = (k + 0.5) * s
    X[:, ::64] = 7.0 * s[:, ::64]  # group max 7 s -> scale exactly s
    bits = bf16_to_bits(X)
    nudge = rng.integers(-1, 2, (M, K)).astype(np.int32)
    nudge[:, ::64] = 0
    bits = (bits.astype(np.int32) + nudge).astype(np.uint16)
    inv = np.ones(K, np.float32)
    ref = osq.quantize_act(bits, inv, None)
    xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    B.svdq_quantize_act(dev_bf16(bits), dev(inv), None, 0, xq, xs, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), ref["xq"])
    assert (nudge == 0).sum() > M * K // 4  # many exact ties were exercised


# (37, 6144, 72, 32) and (65, 6208, 40, 16): K / 64 = 96 and 97, where the activation pass
# splits each row block's groups over two workgroups (97: halves of 49 and 48 groups)
@pytest.mark.parametrize("M,K,N,r", [(1, 64, 24, 16), (17, 192, 136, 32), (129, 320, 129, 48),
                                     (7, 128, 1, 0), (300, 576, 260, 128),
                                     (37, 6144, 72, 32), (65, 6208, 40, 16)])
def test_ragged_shapes_with_guard_bands(gpu_lib, M, K, N, r):
    d = make_linear(3, M=M, K=K, N=N, with_bias=True)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, r)
    packed = osq.pack_weights(pw["R32"])
    ref = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
    G = K // 64
    GUARD = 0x5A
    wq = torch.full((N + 1, K // 2), GUARD, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(G * N + 8, dtype=torch.float16, device="cuda")
    B.svdq_pack_weights(dev(pw["R32"]), wq[:N], ws[:G * N].view(G, N))
    xq = torch.full((M + 1, K // 2), GUARD, dtype=torch.uint8, device="cuda")
    xs = torch.full((G * M + 8,), -3.0, dtype=torch.float16, device="cuda")
    T = torch.full((M + 1, max(r, 1)), -7.0, dtype=torch.float32, device="cuda")
    L1t = dev_bf16(bf16_to_bits(pw["L1b"].T)) if r else None
    L2t = dev_bf16(np.ascontiguousarray(bf16_to_bits(pw["L2b"]).T)) if r else None  # [N, r]
    Tv = T[:M] if r else None
    B.svdq_quantize_act(dev_bf16(d["X"]), dev(pw["inv_lambda"]), L1t, r, xq[:M],
                        xs[:G * M].view(M, G), Tv)
    Y = torch.full((M + 1, N), 3.0, dtype=torch.bfloat16, device="cuda")
    B.svdq_w4a4_gemm(xq[:M], xs[:G * M].view(M, G), Tv, wq[:N], ws[:G * N].view(G, N), L2t,
                     dev_bf16(d["bias"]), r, Y[:M])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wq[:N].cpu().numpy(), packed["wq"])
    np.testing.assert_array_equal(xq[:M].cpu().numpy(), ref["xq"])
    # guard bands untouched
    assert (wq[N].cpu() == GUARD).all() and (xq[M].cpu() == GUARD).all()
    assert (xs[G * M:].cpu() == -3.0).all() and (ws[G * N:].cpu() == 0).all()
    assert (Y[M].cpu().float() == 3.0).all()
    if r:
        assert (T[M].cpu() == -7.0).all()
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                              ref["T"], pw["L2b"], d["bias"])
    assert max_abs_rel(Y[:M].float().cpu().numpy().astype(np.float64), Y_ref) <= TOL


def test_fp32_output_and_determinism(gpu_lib):
    case = _case("c2s", bias=True)
    d, pw, packed, r = case
    w = device_weights(case)
    M, N = d["X"].shape[0], pw["R32"].shape[1]
    wq, ws = _gpu_pack(case)
    xq, xs, T = _gpu_act(case)
    Ya = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Yb = torch.empty(M, N, dtype=torch.float32, device="cuda")
    B.svdq_w4a4_gemm(xq, xs, T, wq, ws, w["L2p"], w["bias"], r, Ya)
    xq2, xs2, T2 = _gpu_act(case)
    B.svdq_w4a4_gemm(xq2, xs2, T2, wq, ws, w["L2p"], w["bias"], r, Yb)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb) and torch.equal(T, T2)
    ref = oracle_act(case)
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                              ref["T"], pw["L2b"], d["bias"])
    assert max_abs_rel(Ya.cpu().numpy().astype(np.float64), Y_ref) <= TOL


# ------------------------------------------------------------------------------- KV cache
def _gpu_kv(x_bits):
    T_, C = x_bits.shape
    x = dev_bf16(x_bits)
    q = torch.empty(T_, C, dtype=torch.uint8, device="cuda")
    s = torch.empty(C, dtype=torch.float32, device="cuda")
    z = torch.empty(C, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(B.kv_int8_workspace_bytes(T_, C), 16), dtype=torch.uint8, device="cuda")
    B.kv_int8_quant(x, q, s, z, ws)
    out = torch.empty(T_, C, dtype=torch.bfloat16, device="cuda")
    B.kv_int8_dequant(q, s, z, out)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy(), host_u16(out)


# (None,)*3 is the full cache [10240, 32, 128] (single pass, 32 slabs of 128 channels);
# (2000, 16, 128) is a single pass over 16 slabs, (1000, 8, 64) over 4 and (300, 3, 128) over 3;
# 1000 and 100 tokens end in a partial 64-token range chunk of the three-pass schedule; 12800
# tokens (three passes) fill 200 chunks; (1, 2, 8) is a single token of 16 channels; (5, 2, 128)
# is a single pass in which some token parts are empty; 2097120 tokens is the most one call
# takes (65535 dequantization blocks of 32 tokens; three passes over 32768 range chunks)
# (1001, 32, 128) and (37, 64, 128): the cache's row width and twice it, with a partial last
# block of the dequantization (32 tokens)
@pytest.mark.parametrize("shape", [(None, None, None), (1, 2, 8), (100, 4, 24), (1000, 8, 64),
                                   (2000, 16, 128), (5, 2, 128), (300, 3, 128), (12800, 32, 128),
                                   (2097120, 1, 8), (1001, 32, 128), (37, 64, 128)])
def test_kv_quant_dequant_bitexact(gpu_lib, shape):
    for name, (x, ref) in kv_case(*shape).items():
        q, s, z, xo = _gpu_kv(x)
        np.testing.assert_array_equal(s.view(np.uint32), ref["scale"].view(np.uint32))
        np.testing.assert_array_equal(z, ref["zero"])
        np.testing.assert_array_equal(q, ref["q"])
        bits, _ = okv.dequantize(ref["q"], ref["scale"], ref["zero"])
        np.testing.assert_array_equal(xo, bits)


def test_kv_workspace_needs_no_initialization_and_is_reusable(gpu_lib):
    """A garbage-filled workspace, reused across tensors of different shapes, gives exact codes."""
    ws = torch.full((B.kv_int8_workspace_bytes(12800, 4096),), 0xA5, dtype=torch.uint8, device="cuda")
    for shape in [(300, 4, 32), (64, 2, 16), (12800, 32, 128), (300, 4, 32)]:
        x, ref = kv_case(*shape)["V"]
        T_, C = x.shape
        q = torch.empty(T_, C, dtype=torch.uint8, device="cuda")
        s = torch.empty(C, dtype=torch.float32, device="cuda")
        z = torch.empty(C, dtype=torch.uint8, device="cuda")
        B.kv_int8_quant(dev_bf16(x), q, s, z, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q.cpu().numpy(), ref["q"])
        np.testing.assert_array_equal(z.cpu().numpy(), ref["zero"])


@pytest.mark.parametrize("shape", [(1000, 8, 64), (10240, 32, 128), (5, 2, 128)])
def test_kv_single_pass_self_contained_path(gpu_lib, shape, monkeypatch):
    """The single-pass quantizer with its bounded wait forced to time out at once: every block
    computes its slabs' ranges from x itself.  Same codes as the oracle; (5, 2, 128) has token
    parts that are empty."""
    monkeypatch.setenv("SVDQ_KV_SPIN_TICKS", "0")
    for name, (x, ref) in kv_case(*shape).items():
        q, s, z, xo = _gpu_kv(x)
        np.testing.assert_array_equal(q, ref["q"])
        np.testing.assert_array_equal(z, ref["zero"])
        np.testing.assert_array_equal(s.view(np.uint32), ref["scale"].view(np.uint32))


def test_kv_repeated_calls_share_a_workspace(gpu_lib):
    """Back-to-back single-pass calls (K, V, K, ...) on one workspace, no synchronization between
    them: each call's exchange only accepts its own partial ranges."""
    case = kv_case(1000, 8, 64)
    ws = torch.full((B.kv_int8_workspace_bytes(1000, 512),), 0xA5, dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(3):
        for name in ("K", "V"):
            x, ref = case[name]
            q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
            s = torch.empty(x.shape[1], dtype=torch.float32, device="cuda")
            z = torch.empty(x.shape[1], dtype=torch.uint8, device="cuda")
            B.kv_int8_quant(dev_bf16(x), q, s, z, ws)
            outs.append((name, q, z))
    torch.cuda.synchronize()
    for name, q, z in outs:
        np.testing.assert_array_equal(q.cpu().numpy(), case[name][1]["q"])
        np.testing.assert_array_equal(z.cpu().numpy(), case[name][1]["zero"])


def test_kv_degenerate_channels(gpu_lib):
    T_, C = 70, 32
    x = np.random.default_rng(13).standard_normal((T_, C))
    x[:, 0] = 0.0               # constant zero channel -> s = 1, z = 0
    x[:, 1] = np.abs(x[:, 1])   # all non-negative -> z = 0
    x[:, 2] = -np.abs(x[:, 2])  # all non-positive -> z = 255
    x[:, 3] = 1.5               # constant positive channel
    bits = bf16_to_bits(round_bf16(x))
    ref = okv.kv_int8_quant(bits)
    q, s, z, xo = _gpu_kv(bits)
    np.testing.assert_array_equal(q, ref["q"])
    np.testing.assert_array_equal(z, ref["zero"])
    np.testing.assert_array_equal(s.view(np.uint32), ref["scale"].view(np.uint32))
    assert s[0] == 1.0 and z[0] == 0 and z[1] == 0 and z[2] == 255
