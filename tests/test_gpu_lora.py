"""GPU parity of a LoRA adapter attached to the 16-bit branch (SVDQ "feature list": adapters
integrate without re-quantization): the packed residual is reused as it is, the branch grows to
rank r + r_l, and both code containers still match the oracle -- activation codes and scales
bit-exact, T and Y within the output tolerance."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits
from tests.gpu_cases import dev, dev_bf16, host_u16, linear_case, max_abs_rel, pack_l2

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.mark.parametrize("rl", [16, 32, 96])    # combined rank 48, 64 and the maximum 128
@pytest.mark.parametrize("e3m2", [False, True])
def test_lora_branch_parity(gpu_lib, rl, e3m2):
    case = linear_case(2, 300, 512, 384, True)
    d, pw, packed, r = case
    M, K = d["X"].shape
    N = pw["R32"].shape[1]
    rng = np.random.default_rng(rl)
    A = rng.standard_normal((K, rl)) / np.sqrt(K)
    Bm = rng.standard_normal((rl, N)) * 0.2
    L1p, L2p = osq.attach_lora(pw["L1b"], pw["L2b"], pw["lam32"], A, Bm, 0.5)
    r2 = r + rl
    ref = osq.quantize_act(d["X"], pw["inv_lambda"], L1p)
    Y_ref = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"], ref["T"],
                              L2p, d["bias"])

    L1t = dev_bf16(bf16_to_bits(L1p.T))
    L2t = pack_l2(dev_bf16(bf16_to_bits(L2p)))  # [r, N] -> [N, r]
    inv = dev(pw["inv_lambda"])
    R32 = dev(pw["R32"])
    bias = dev_bf16(d["bias"])
    ws = torch.empty(K // 64, N, dtype=torch.float16, device="cuda")
    xs = torch.empty(M, K // 64, dtype=torch.float16, device="cuda")
    T = torch.empty(M, r2, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    X = dev_bf16(d["X"])
    if e3m2:
        wq = torch.empty(B.svdq_e3m2_bytes(N, K), dtype=torch.uint8, device="cuda")
        xq = torch.empty(B.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device="cuda")
        B.svdq_pack_weights_e3m2(R32, wq, ws)
        B.svdq_quantize_act_e3m2(X, inv, L1t, r2, xq, xs, T)
        B.svdq_w4a4_gemm_e3m2(xq, xs, T, wq, ws, L2t, bias, r2, Y)
        want_xq = osq.pack_e3m2_tiled(ref["codes"]).reshape(-1)
    else:
        wq = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
        xq = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
        B.svdq_pack_weights(R32, wq, ws)
        B.svdq_quantize_act(X, inv, L1t, r2, xq, xs, T)
        B.svdq_w4a4_gemm(xq, xs, T, wq, ws, L2t, bias, r2, Y)
        want_xq = ref["xq"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), want_xq)
    np.testing.assert_array_equal(host_u16(xs), np.ascontiguousarray(ref["s_x"]).view(np.uint16))
    assert max_abs_rel(T.cpu().numpy().astype(np.float64), ref["T"]) <= TOL
    assert max_abs_rel(Y.float().cpu().numpy().astype(np.float64), Y_ref) <= TOL
    # the adapter really changed the output (its term is not lost in the tolerance)
    Y_base = osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"],
                               ref["T"][:, :r], pw["L2b"], d["bias"])
    assert max_abs_rel(Y_base, Y_ref) > 10 * TOL
