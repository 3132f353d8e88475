"""Host side of LoRA attachment: layer.attach_lora builds exactly the oracle's extended branch
factors (bit-identical bf16), keeps the packed residual, and validates shapes and ranks."""
import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding, layer
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, round_bf16
from synthetic import make_linear


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _packed(pw, r):
    K, N = pw["R32"].shape
    return layer.PackedWeights(
        K=K, N=N, rank=r, inv_lambda=torch.from_numpy(pw["inv_lambda"]),
        L1p=torch.from_numpy(bf16_to_bits(pw["L1b"].T).view(np.int16)).view(torch.bfloat16),
        L2p=torch.from_numpy(bf16_to_bits(pw["L2b"].T).view(np.int16)).view(torch.bfloat16),
        wq=torch.zeros(1, dtype=torch.uint8), w_scales=torch.zeros(1, dtype=torch.float16),
        lam=torch.from_numpy(pw["lam32"]))


def _host_transpose(src, dst):
    """Host stand-in for the device relayouts (the library needs a GPU): dst = src^T."""
    dst.copy_(src.t())


@pytest.mark.parametrize("rl,scale", [(16, 1.0), (32, 0.375)])
def test_attach_lora_matches_the_oracle_bit_for_bit(rl, scale, monkeypatch):
    monkeypatch.setattr(binding, "svdq_pack_lowrank", _host_transpose)
    monkeypatch.setattr(binding, "svdq_pack_lowrank_up", _host_transpose)
    d = make_linear(2, M=40, K=256, N=80, seed=3)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, 16)
    rng = np.random.default_rng(9)
    A = rng.standard_normal((256, rl)) / 16
    B = rng.standard_normal((rl, 80)) * 0.3
    L1p, L2p = osq.attach_lora(pw["L1b"], pw["L2b"], pw["lam32"], A, B, scale)
    base = _packed(pw, 16)
    out = layer.attach_lora(base, torch.from_numpy(A), torch.from_numpy(B), scale)
    assert out.rank == 16 + rl
    np.testing.assert_array_equal(_bits(out.L1p), bf16_to_bits(L1p.T))
    np.testing.assert_array_equal(_bits(out.L2p), bf16_to_bits(L2p.T))
    assert out.wq is base.wq and out.w_scales is base.w_scales  # no re-quantization


def test_attach_lora_rejects_bad_ranks_and_shapes():
    d = make_linear(2, M=40, K=256, N=80, seed=3)
    pw = _packed(osq.prepare_weights(d["X"], d["W"], 0.5, 16), 16)
    with pytest.raises(ValueError):
        layer.attach_lora(pw, torch.zeros(256, 8), torch.zeros(8, 80))      # 24: not /16
    with pytest.raises(ValueError):
        layer.attach_lora(pw, torch.zeros(256, 128), torch.zeros(128, 80))  # 144 > 128
    with pytest.raises(ValueError):
        layer.attach_lora(pw, torch.zeros(255, 16), torch.zeros(16, 80))    # K mismatch
