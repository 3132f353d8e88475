"""The product path through layer.py on the GPU: the factor relayouts (svdq_pack_lowrank,
svdq_pack_lowrank_up) bit-exact, and layer.pack_device + layer.forward -- the calls bench.py times -- at the full
FFN up-projection shape, every output row against the oracle's fp64 output.

The host half of the weight preparation (layer.prepare_host) is pinned against the oracle on
the CPU (tests/test_layer_host.py); here the device half starts from the oracle's prepared
weights, so both sides quantize the same residual."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import layer
from oracle.numerics import bf16_to_bits
from tests.gpu_cases import dev_bf16, host_u16, linear_case, max_abs_rel, oracle_output

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.mark.parametrize("K,r", [(64, 16), (256, 16), (3072, 32), (12288, 32), (320, 48),
                                 (192, 128)])
def test_pack_lowrank_bitexact(gpu_lib, K, r):
    rng = np.random.default_rng(K + r)
    bits = rng.integers(0, 1 << 16, (K, r), dtype=np.uint32).astype(np.uint16)
    L1p = layer.pack_lowrank(dev_bf16(bits))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(L1p), np.ascontiguousarray(bits.T))


@pytest.mark.parametrize("r,N", [(16, 64), (16, 1), (32, 12288), (32, 3072), (48, 200),
                                 (128, 130)])
def test_pack_lowrank_up_bitexact(gpu_lib, r, N):
    rng = np.random.default_rng(r * 7 + N)
    bits = rng.integers(0, 1 << 16, (r, N), dtype=np.uint32).astype(np.uint16)
    L2p = layer.pack_lowrank_up(dev_bf16(bits))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(L2p), np.ascontiguousarray(bits.T))


def _host_weights(pw):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    bf = lambda a: t(bf16_to_bits(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    return layer.HostWeights(lam=t(pw["lam32"]), inv_lambda=t(pw["inv_lambda"]),
                             L1b=bf(pw["L1b"]), L2b=bf(pw["L2b"]), R32=t(pw["R32"]))


@pytest.mark.parametrize("e3m2,bias", [(True, False), (True, True), (False, False)])
def test_layer_forward_full_ffn_up(gpu_lib, e3m2, bias):
    d, pw, packed, r = linear_case(3, None, None, None, bias)
    b = dev_bf16(d["bias"]) if bias else None
    pwd = layer.pack_device(_host_weights(pw), b, e3m2=e3m2)
    Y = layer.forward(dev_bf16(d["X"]), pwd)
    torch.cuda.synchronize()
    Y_ref = oracle_output(3, None, None, None, d["bias"])
    err = max_abs_rel(Y.float().cpu().numpy().astype(np.float64), Y_ref)
    assert err <= TOL, err
