"""SVDQuant linear layer on top of the C ABI: offline weight conversion and the forward pass.

Weight conversion (offline, host): the three steps of SVDQuant (SVDQ "technical principles";
FLUX4 2.2) — smoothing factors from calibration activations, a rank-r SVD of the smoothed
weight kept as a bf16 low-rank branch, and the fp32 residual, which ``svdq_pack_weights``
quantizes to packed INT4 on the device.  The SVD is a LAPACK call through torch on the host:
it is the offline preparation a toolbox performs once per checkpoint, not part of the
per-token path.

Forward (device): ``svdq_quantize_act`` then ``svdq_w4a4_gemm``, two launches on one stream.
The factors are relaid out once, like the residual: L1 [K, r] to the activation pass's
[r, K] by ``svdq_pack_lowrank``, L2 [r, N] to the GEMM epilogue's [N, r] by
``svdq_pack_lowrank_up``.
With ``e3m2=True`` the codes travel as BF6 (E3M2) values and the ``*_e3m2`` entry points run
the GEMM on the FP6 matrix units (same codes, scales and result; the faster path on gfx950).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import torch

from . import binding


@dataclass
class PackedWeights:
    K: int
    N: int
    rank: int
    inv_lambda: torch.Tensor  # fp32 [K]
    L1p: torch.Tensor         # bf16 [r, K]  (the [K, r] factor, from svdq_pack_lowrank)
    L2p: torch.Tensor         # bf16 [N, r]  (the [r, N] factor, from svdq_pack_lowrank_up)
    wq: torch.Tensor          # uint8 [N, K/2] (nibbles) or the tiled BF6 container of N rows
    w_scales: torch.Tensor    # fp16 [K/64, N]
    bias: Optional[torch.Tensor] = None  # bf16 [N]
    e3m2: bool = False        # container of wq (and of the activation codes in forward)
    R32: Optional[torch.Tensor] = None  # fp32 [K, N] residual, kept only on request
    lam: Optional[torch.Tensor] = None  # fp32 [K] smoothing factors (host), for adapters


def _bf16_rn(x: torch.Tensor) -> torch.Tensor:
    """float64 -> bf16 with one round-to-nearest-even: round to odd into fp32 (24 bits keep
    the two extra bits that make the second rounding exact), then fp32 -> bf16 (RNE)."""
    x = x.to(torch.float64)
    t = x.to(torch.float32)
    over = t.to(torch.float64).abs() > x.abs()
    t = torch.where(over, torch.nextafter(t, torch.zeros_like(t)), t)  # toward zero
    inexact = (t.to(torch.float64) != x).to(torch.int32)
    return (t.view(torch.int32) | inexact).view(torch.float32).to(torch.bfloat16)


@dataclass
class HostWeights:
    """The offline host half of the weight conversion (all CPU tensors)."""
    lam: torch.Tensor         # fp32 [K] smoothing factors
    inv_lambda: torch.Tensor  # fp32 [K] = fl32(1 / lam)
    L1b: torch.Tensor         # bf16 [K, r]
    L2b: torch.Tensor         # bf16 [r, N]
    R32: torch.Tensor         # fp32 [K, N] residual W^ - L1b L2b


def prepare_host(W: torch.Tensor, X_calib: torch.Tensor, alpha: float, rank: int) -> HostWeights:
    """Smoothing factors from the calibration activations, the rank-r split of the smoothed
    weight kept in bf16, and the fp32 residual (SVDQ "technical principles"; FLUX4 2.2).

    W bf16 [K, N] (Y = X W), X_calib bf16 [M, K].  lam_k = max|X_k|^alpha / max|W_k|^(1-alpha)
    (1 where either is 0), W^ = diag(lam32) W in fp64, L1 = U_r S_r and L2 = V_r^T rounded once
    to bf16, R = W^ - L1b L2b in fp64 stored as fp32."""
    K, N = W.shape
    Wd = W.detach().to("cpu", torch.float64)
    Xd = X_calib.detach().to("cpu", torch.float64)
    a = Xd.abs().amax(dim=0) if Xd.shape[0] else torch.zeros(K, dtype=torch.float64)
    w = Wd.abs().amax(dim=1)
    ok = (a > 0) & (w > 0)
    lam = torch.ones(K, dtype=torch.float64)
    lam[ok] = a[ok].pow(alpha) / w[ok].pow(1.0 - alpha)
    lam32 = lam.to(torch.float32)
    inv32 = torch.ones(K, dtype=torch.float32) / lam32
    W_hat = lam32.to(torch.float64)[:, None] * Wd
    if rank > 0:
        U, S, Vh = torch.linalg.svd(W_hat, full_matrices=False)
        L1b = _bf16_rn(U[:, :rank] * S[:rank])
        L2b = _bf16_rn(Vh[:rank, :])
        R = W_hat - L1b.to(torch.float64) @ L2b.to(torch.float64)
    else:
        L1b = torch.zeros(K, 0, dtype=torch.bfloat16)
        L2b = torch.zeros(0, N, dtype=torch.bfloat16)
        R = W_hat
    return HostWeights(lam=lam32, inv_lambda=inv32, L1b=L1b, L2b=L2b,
                       R32=R.to(torch.float32).contiguous())


def pack_device(hw: HostWeights, bias: Optional[torch.Tensor] = None, device="cuda",
                e3m2: bool = False, keep_residual: bool = False) -> PackedWeights:
    """The device half of the weight conversion: the residual's INT4 codes and scales
    (``svdq_pack_weights``, or ``svdq_pack_weights_e3m2`` for the BF6 container) and the factor
    relayouts (``svdq_pack_lowrank``, ``svdq_pack_lowrank_up``)."""
    K, N = hw.R32.shape
    rank = hw.L1b.shape[1]
    R32 = hw.R32.to(device).contiguous()
    w_scales = torch.empty(K // 64, N, dtype=torch.float16, device=device)
    if e3m2:
        wq = torch.empty(binding.svdq_e3m2_bytes(N, K), dtype=torch.uint8, device=device)
        binding.svdq_pack_weights_e3m2(R32, wq, w_scales)
    else:
        wq = torch.empty(N, K // 2, dtype=torch.uint8, device=device)
        binding.svdq_pack_weights(R32, wq, w_scales)
    return PackedWeights(
        K=K, N=N, rank=rank, inv_lambda=hw.inv_lambda.to(device),
        L1p=pack_lowrank(hw.L1b.to(device)), L2p=pack_lowrank_up(hw.L2b.to(device)),
        wq=wq, w_scales=w_scales,
        bias=None if bias is None else bias.to(device, torch.bfloat16).contiguous(), e3m2=e3m2,
        R32=R32 if keep_residual else None, lam=hw.lam)


def convert_weights(W: torch.Tensor, X_calib: torch.Tensor, alpha: float, rank: int,
                    bias: Optional[torch.Tensor] = None, device="cuda",
                    e3m2: bool = False, keep_residual: bool = False) -> PackedWeights:
    """W bf16 [K, N] (Y = X W), X_calib bf16 [M, K] calibration activations: ``prepare_host``
    then ``pack_device``."""
    return pack_device(prepare_host(W, X_calib, alpha, rank), bias, device, e3m2, keep_residual)


def pack_lowrank(L1: torch.Tensor) -> torch.Tensor:
    """L1 bf16 [K, r] on the device -> L1p [r, K] (``svdq_pack_lowrank``); [0, K] for r = 0."""
    K, r = L1.shape
    L1p = torch.empty(r, K, dtype=torch.bfloat16, device=L1.device)
    if r:
        binding.svdq_pack_lowrank(L1.contiguous(), L1p)
    return L1p


def pack_lowrank_up(L2: torch.Tensor) -> torch.Tensor:
    """L2 bf16 [r, N] on the device -> L2p [N, r] (``svdq_pack_lowrank_up``); [N, 0] for r = 0."""
    r, N = L2.shape
    L2p = torch.empty(N, r, dtype=torch.bfloat16, device=L2.device)
    if r:
        binding.svdq_pack_lowrank_up(L2.contiguous(), L2p)
    return L2p


def attach_lora(pw: PackedWeights, A: torch.Tensor, B: torch.Tensor,
                scale: float = 1.0) -> PackedWeights:
    """Attach a low-rank adapter W' = W + scale * A B (A [K, r_l], B [r_l, N]) to the 16-bit
    branch without re-quantizing the 4-bit residual (SVDQ "feature list": LoRA adapters
    integrate without re-quantization).

    The branch runs on X^ = X diag(lam)^-1, so the adapter joins it as extra rank in the smoothed
    frame: L1' = [L1 | bf16(lam * A)], L2' = [L2 ; bf16(scale * B)].  The packed codes and
    scales are shared with ``pw``; the combined rank must stay a multiple of 16, at most 128.
    """
    if pw.lam is None:
        raise ValueError("attach_lora needs the smoothing factors (weights from convert_weights)")
    K, rl = A.shape
    if K != pw.K or B.shape != (rl, pw.N):
        raise ValueError(f"adapter shapes {tuple(A.shape)} x {tuple(B.shape)} do not fit K={pw.K}, N={pw.N}")
    r2 = pw.rank + rl
    if r2 % 16 or r2 > 128:
        raise ValueError(f"combined rank {r2} must be a multiple of 16 and at most 128")
    dev = pw.L1p.device
    A_hat = _bf16_rn(pw.lam.to("cpu", torch.float64)[:, None] * A.to("cpu", torch.float64))
    B_s = _bf16_rn(scale * B.to("cpu", torch.float64))
    L1p = torch.cat([pw.L1p, pack_lowrank(A_hat.to(dev))], dim=0).contiguous()
    L2p = torch.cat([pw.L2p, pack_lowrank_up(B_s.to(dev))], dim=1).contiguous()
    return dataclasses.replace(pw, rank=r2, L1p=L1p, L2p=L2p)


@dataclass
class ActBuffers:
    xq: torch.Tensor
    x_scales: torch.Tensor
    T: Optional[torch.Tensor]


def alloc_act(M: int, K: int, rank: int, device="cuda", e3m2: bool = False) -> ActBuffers:
    return ActBuffers(
        xq=(torch.empty(binding.svdq_e3m2_bytes(M, K), dtype=torch.uint8, device=device) if e3m2
            else torch.empty(M, K // 2, dtype=torch.uint8, device=device)),
        x_scales=torch.empty(M, K // 64, dtype=torch.float16, device=device),
        T=torch.empty(M, rank, dtype=torch.float32, device=device) if rank > 0 else None)


def forward(X: torch.Tensor, pw: PackedWeights, out: Optional[torch.Tensor] = None,
            act: Optional[ActBuffers] = None, out_dtype=torch.bfloat16,
            stream=None) -> torch.Tensor:
    """Y = SVDQuant-linear(X) for X bf16 [M, K] on the device."""
    M, K = X.shape
    if act is None:
        act = alloc_act(M, K, pw.rank, X.device, pw.e3m2)
    if out is None:
        out = torch.empty(M, pw.N, dtype=out_dtype, device=X.device)
    quantize = binding.svdq_quantize_act_e3m2 if pw.e3m2 else binding.svdq_quantize_act
    gemm = binding.svdq_w4a4_gemm_e3m2 if pw.e3m2 else binding.svdq_w4a4_gemm
    quantize(X, pw.inv_lambda, pw.L1p if pw.rank else None, pw.rank, act.xq, act.x_scales,
             act.T, stream)
    gemm(act.xq, act.x_scales, act.T, pw.wq, pw.w_scales, pw.L2p if pw.rank else None,
         pw.bias, pw.rank, out, stream)
    return out
