"""GPU parity of kv_int8_quant_pair: K and V of one layer quantized in one launch must give the
oracle's codes, scales and zero points for each tensor, bit for bit, on every schedule the call
can take (the paired single pass, its bounded wait timed out, and two three-pass calls)."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from tests.gpu_cases import dev_bf16, kv_case

pytestmark = pytest.mark.gpu


def _outs(T_, C):
    return [torch.empty(T_, C, dtype=torch.uint8, device="cuda"),
            torch.empty(C, dtype=torch.float32, device="cuda"),
            torch.empty(C, dtype=torch.uint8, device="cuda")]


def _check(outs, ref):
    q, s, z = (t.cpu().numpy() for t in outs)
    np.testing.assert_array_equal(s.view(np.uint32), ref["scale"].view(np.uint32))
    np.testing.assert_array_equal(z, ref["zero"])
    np.testing.assert_array_equal(q, ref["q"])


def _pair(case, ws=None):
    (xk, rk), (xv, rv) = case["K"], case["V"]
    T_, C = xk.shape
    if ws is None:
        ws = torch.full((max(B.kv_int8_workspace_bytes(T_, C), 16),), 0xA5, dtype=torch.uint8,
                        device="cuda")
    ok, ov = _outs(T_, C), _outs(T_, C)
    B.kv_int8_quant_pair(dev_bf16(xk), dev_bf16(xv), *ok, *ov, ws)
    return ok, ov


# (None,)*3 is the full cache [10240, 32, 128]: the paired single pass over 32 slabs with 40 rows
# per thread; (2000, 16, 128) pairs over 16 slabs; (300, 3, 128) over 3 slabs (parts not grouped
# by XCD); (5, 2, 128) has empty token parts; (100, 4, 24) and (12800, 32, 128) are shapes the
# single pass does not take (two three-pass calls); (1, 2, 8) is one token of 16 channels
@pytest.mark.parametrize("shape", [(None, None, None), (2000, 16, 128), (300, 3, 128),
                                   (5, 2, 128), (100, 4, 24), (12800, 32, 128), (1, 2, 8)])
def test_pair_matches_the_oracle(gpu_lib, shape):
    case = kv_case(*shape)
    ok, ov = _pair(case)
    torch.cuda.synchronize()
    _check(ok, case["K"][1])
    _check(ov, case["V"][1])


@pytest.mark.parametrize("shape", [(None, None, None), (5, 2, 128)])
def test_pair_self_contained_path(gpu_lib, shape, monkeypatch):
    """The bounded wait forced to time out at once: every block computes both tensors' ranges
    from x itself."""
    monkeypatch.setenv("SVDQ_KV_SPIN_TICKS", "0")
    case = kv_case(*shape)
    ok, ov = _pair(case)
    torch.cuda.synchronize()
    _check(ok, case["K"][1])
    _check(ov, case["V"][1])


def test_pair_and_single_calls_share_a_workspace(gpu_lib):
    """Paired and single calls back to back on one garbage-filled workspace, no synchronization
    between them: each exchange accepts only its own call's partial ranges."""
    case = kv_case(1000, 8, 64)
    T_, C = case["K"][0].shape
    ws = torch.full((B.kv_int8_workspace_bytes(T_, C),), 0x5A, dtype=torch.uint8, device="cuda")
    runs = []
    for rep in range(3):
        runs.append(("pair",) + _pair(case, ws))
        single = _outs(T_, C)
        B.kv_int8_quant(dev_bf16(case["V"][0]), *single, ws)
        runs.append(("V", single))
    torch.cuda.synchronize()
    for run in runs:
        if run[0] == "pair":
            _check(run[1], case["K"][1])
            _check(run[2], case["V"][1])
        else:
            _check(run[1], case["V"][1])


def test_pair_equals_two_single_calls_on_distinct_inputs(gpu_lib):
    """K and V drawn from different seeds (different ranges per channel): the pair gives each
    tensor its own parameters, identical to two kv_int8_quant calls."""
    a, b = kv_case(2000, 16, 128, seed=3), kv_case(2000, 16, 128, seed=4)
    case = {"K": a["V"], "V": b["K"]}
    ok, ov = _pair(case)
    T_, C = case["K"][0].shape
    ws = torch.empty(B.kv_int8_workspace_bytes(T_, C), dtype=torch.uint8, device="cuda")
    sk, sv = _outs(T_, C), _outs(T_, C)
    B.kv_int8_quant(dev_bf16(case["K"][0]), *sk, ws)
    B.kv_int8_quant(dev_bf16(case["V"][0]), *sv, ws)
    torch.cuda.synchronize()
    for x, y in zip(ok + ov, sk + sv):
        assert torch.equal(x, y)
    _check(ok, case["K"][1])
    _check(ov, case["V"][1])
