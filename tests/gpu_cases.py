"""Shared inputs for the GPU parity tests: seeded workloads, the oracle's prepared weights and
device copies in the layouts of include/svdq.h.  (Not a test module.)"""
from __future__ import annotations

import functools

import numpy as np
import torch

from oracle import kv_int8 as okv
from oracle import svdquant as osq
from oracle.numerics import bf16_to_bits, decode_bf16
from synthetic import LINEAR_CONFIGS, make_bias, make_kv, make_linear

# (config id, M, K, N): small cases that span several 128x128 tiles with ragged tails, and the
# full workload shapes (which run in the same launch configuration as the benchmark)
SMALL = {
    "c1": (1, None, None, None),
    "c2s": (2, 300, 512, 384),
    "c3s": (3, 257, 1024, 640),
    "c4s": (4, 130, 2048, 200),
}
FULL = {"c2": (2, None, None, None), "c3": (3, None, None, None), "c4": (4, None, None, None)}


def with_bias(cases):
    """(name, bias) pairs for the output tests: bias at the small shapes and at the FFN-up
    shape (the benchmark's), none at the other full shapes."""
    return [(n, b) for n in cases for b in (False, True) if not (b and n in FULL and n != "c3")]


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=None)
def _base_case(cid: int, M, K, N):
    d = make_linear(cid, M=M, K=K, N=N)
    cfg = LINEAR_CONFIGS[cid]
    pw = osq.prepare_weights(d["X"], d["W"], cfg.alpha, cfg.rank)
    packed = osq.pack_weights(pw["R32"])
    return d, pw, packed, cfg.rank


def linear_case(cid: int, M, K, N, bias: bool = False):
    """Workload + the oracle's weight preparation and packed weights (cached per session; the
    bias case shares X, W and the prepared weights of the case without bias)."""
    d, pw, packed, r = _base_case(cid, M, K, N)
    if bias:
        d = dict(d, bias=make_bias(cid, pw["R32"].shape[1]))
    return d, pw, packed, r


@functools.lru_cache(maxsize=None)
def _oracle_output(cid: int, M, K, N):
    d, pw, packed, r = _base_case(cid, M, K, N)
    ref = oracle_act((d, pw, packed, r))
    return osq.linear_output(ref["codes"], ref["s_x"], packed["codes"], packed["s_w"], ref["T"],
                             pw["L2b"], None)


def oracle_output(cid: int, M, K, N, bias=None):
    """The oracle's Y of the whole workload (every row; fp64), plus the bias when given."""
    Y = _oracle_output(cid, M, K, N)
    return Y if bias is None else Y + decode_bf16(bias)[None, :]


def oracle_act(case):
    d, pw, _, _ = case
    return osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])


def pack_l2(L2):
    """L2 [r, N] on the device -> L2p [N, r] through the library's relayout."""
    from bit_post_quantized_amd import layer
    return layer.pack_lowrank_up(L2)


def device_weights(case):
    """Oracle-prepared weights in the C-ABI layouts on the device."""
    d, pw, packed, r = case
    return dict(
        inv_lambda=dev(pw["inv_lambda"]),
        L1p=dev_bf16(bf16_to_bits(pw["L1b"].T)) if r else None,  # [r, K]
        L2p=pack_l2(dev_bf16(bf16_to_bits(pw["L2b"]))) if r else None,  # [N, r]
        R32=dev(pw["R32"]),
        bias=dev_bf16(d["bias"]) if d["bias"] is not None else None,
    )


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref|: the output tolerance metric (normwise)."""
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


@functools.lru_cache(maxsize=None)
def kv_case(tokens=None, heads=None, dim=None, seed=0):
    d = make_kv(seed=seed, tokens=tokens, heads=heads, dim=dim)
    out = {}
    for name in ("K", "V"):
        x = d[name].reshape(d[name].shape[0], -1)
        out[name] = (x, okv.kv_int8_quant(x))
    return out
