"""kv_int8_quant_pair_noalloc (the paired KV quantizer on the library's own device scratch)
against kv_int8_quant_pair with a caller-owned workspace, through the C ABI: codes, scales and
zero points bit for bit, on calls in a row whose sizes shrink, so that each call runs on what
the previous one left in the scratch."""
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


# the full cache (paired single pass over 32 slabs), then smaller: 2000 tokens over 16 slabs,
# 100 tokens of 96 channels (three-pass schedule on the scratch), 5 tokens (empty parts)
SEQUENCE = [(None, None, None), (2000, 16, 128), (100, 4, 24), (5, 2, 128)]


def test_noalloc_matches_the_workspace_entry_on_shrinking_calls(gpu_lib):
    for shape in SEQUENCE:
        case = kv_case(*shape)
        (xk, rk), (xv, rv) = case["K"], case["V"]
        T_, C = xk.shape
        k, v = dev_bf16(xk), dev_bf16(xv)
        ws = torch.full((max(B.kv_int8_workspace_bytes(T_, C), 16),), 0xA5, dtype=torch.uint8,
                        device="cuda")
        want_k, want_v = _outs(T_, C), _outs(T_, C)
        B.kv_int8_quant_pair(k, v, *want_k, *want_v, ws)
        got_k, got_v = _outs(T_, C), _outs(T_, C)
        B.kv_int8_quant_pair_noalloc(k, v, *got_k, *got_v)
        torch.cuda.synchronize()
        for g, w in zip(got_k + got_v, want_k + want_v):
            assert torch.equal(g, w), shape
        np.testing.assert_array_equal(got_k[0].cpu().numpy(), rk["q"])
        np.testing.assert_array_equal(got_v[0].cpu().numpy(), rv["q"])


def test_noalloc_back_to_back_without_synchronization(gpu_lib):
    """Two calls queued on one stream with no synchronization between them (the second smaller):
    the second runs on the scratch the first has just used."""
    big, small = kv_case(2000, 16, 128), kv_case(300, 3, 128)
    outs = []
    for case in (big, small):
        T_, C = case["K"][0].shape
        ok, ov = _outs(T_, C), _outs(T_, C)
        B.kv_int8_quant_pair_noalloc(dev_bf16(case["K"][0]), dev_bf16(case["V"][0]), *ok, *ov)
        outs.append((case, ok, ov))
    torch.cuda.synchronize()
    for case, ok, ov in outs:
        np.testing.assert_array_equal(ok[0].cpu().numpy(), case["K"][1]["q"])
        np.testing.assert_array_equal(ov[0].cpu().numpy(), case["V"][1]["q"])
        np.testing.assert_array_equal(ok[2].cpu().numpy(), case["K"][1]["zero"])
        np.testing.assert_array_equal(ov[1].cpu().numpy().view(np.uint32),
                                      case["V"][1]["scale"].view(np.uint32))


def test_noalloc_rejects_shapes_beyond_its_scratch(gpu_lib):
    T_, C = 65536, 4096
    assert B.kv_int8_workspace_bytes(T_, C) > 16 << 20
    k = torch.empty(T_, C, dtype=torch.bfloat16, device="cuda")
    ok, ov = _outs(T_, C), _outs(T_, C)
    with pytest.raises(RuntimeError, match="holds 16777216"):
        B.kv_int8_quant_pair_noalloc(k, k, *ok, *ov)
