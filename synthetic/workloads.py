"""Seeded synthetic inputs for the SVDQuant linear layer and the INT8 KV-cache quantizer.

The pages measure on activations and weights of trained diffusion / visual-autoregressive
models (FLUX.1, Infinity VAR). None of those are available, so these generators stand in for
them: they take the shapes of the five workloads and the distribution statistics the pages
print, and nothing else.

* Activations with a few outlier input channels (the smoothing step exists because of them:
  "SVDQuant technical principles" on the zhuoshang.net SVDQuant overview).
* The FFN down-projection activations of the VAR-Compressor page: heavy-tailed (kurtosis well
  above a Gaussian's) with a max/median magnitude ratio of about 353.
* KV-cache values that are right-skewed (skewness about 0.85) with per-channel spread driven
  by a few channels (coefficient of variation of the channel scale above 1.2), also from the
  VAR-Compressor page ("INT8 KV cache quantization").

Random streams: ``numpy.random.Generator(PCG64(SeedSequence([seed, config_id, tag])))`` with
one tag per tensor, so that every tensor is reproducible on its own. Values are drawn in fp64
and stored as bf16 bit patterns (fp64 -> fp32 -> bf16, each step round-to-nearest-even).

No quantization arithmetic lives here: this module is shared by the CPU oracle and the GPU
path and must stay neutral.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# tensor tags of the random streams
TAG_X, TAG_W, TAG_OUTLIER_CH, TAG_OUTLIER_SCALE, TAG_SPIKE, TAG_BIAS = 1, 2, 3, 4, 5, 6
TAG_K, TAG_V, TAG_CHANNEL_SIGMA = 7, 8, 9


@dataclass(frozen=True)
class LinearConfig:
    """One SVDQuant linear workload: X bf16 [M, K], W bf16 [K, N], rank, group 64."""

    cid: int
    name: str
    M: int
    K: int
    N: int
    rank: int
    alpha: float
    x_model: str  # "gauss" or "laplace"
    n_outliers: Optional[int] = None  # fixed count (else outlier_frac * K)
    outlier_frac: float = 0.0
    outlier_scale: tuple = (100.0, 100.0)  # U[lo, hi]; ignored for "laplace"
    max_median_ratio: Optional[float] = None  # "laplace" target for max|x| / median|x|
    spike_rank: int = 0
    spike_norm: float = 0.0
    group: int = 64


@dataclass(frozen=True)
class KVConfig:
    cid: int
    name: str
    tokens: int
    heads: int
    dim: int
    log_sigma: float = 0.2714  # log-normal shape: skewness (e^{s^2}+2) sqrt(e^{s^2}-1) = 0.8506
    channel_log_std: float = 1.1  # per-channel scale sigma_c = exp(1.1 z_c): CV about 1.5


LINEAR_CONFIGS = {
    1: LinearConfig(1, "tiny", 64, 256, 256, 16, 0.5, "gauss", n_outliers=4,
                    outlier_scale=(100.0, 100.0)),
    2: LinearConfig(2, "attn_proj", 4608, 3072, 3072, 32, 0.5, "gauss", outlier_frac=0.01,
                    outlier_scale=(20.0, 100.0), spike_rank=8, spike_norm=10.0),
    3: LinearConfig(3, "ffn_up", 4608, 3072, 12288, 32, 0.5, "gauss", outlier_frac=0.01,
                    outlier_scale=(20.0, 100.0)),
    4: LinearConfig(4, "ffn_down", 4608, 12288, 3072, 32, 0.5, "laplace", outlier_frac=0.005,
                    max_median_ratio=353.0),
}
KV_CONFIG = KVConfig(5, "kv_cache", 10240, 32, 128)


def make_rng(seed: int, cid: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tag])))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 bit patterns (uint16), both steps round-to-nearest-even."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def _outlier_channels(cfg: LinearConfig, K: int, seed: int) -> np.ndarray:
    n = cfg.n_outliers if cfg.n_outliers is not None else max(1, int(round(cfg.outlier_frac * K)))
    n = min(n, K)
    return np.sort(make_rng(seed, cfg.cid, TAG_OUTLIER_CH).choice(K, size=n, replace=False))


def make_linear(cid: int, seed: int = 0, M: Optional[int] = None, K: Optional[int] = None,
                N: Optional[int] = None, with_bias: bool = False) -> dict:
    """Return {X, W, bias, outlier_channels, cfg, M, K, N} with X/W/bias as bf16 bit patterns.

    X is [M, K] row-major, W is [K, N] row-major (Y = X W). Shapes default to the workload's;
    smaller shapes keep the same distribution model (used for fast parity cases).
    """
    cfg = LINEAR_CONFIGS[cid]
    M = cfg.M if M is None else M
    K = cfg.K if K is None else K
    N = cfg.N if N is None else N
    chans = _outlier_channels(cfg, K, seed)
    rx = make_rng(seed, cid, TAG_X)
    if cfg.x_model == "gauss":
        X = rx.standard_normal((M, K))
        scales = make_rng(seed, cid, TAG_OUTLIER_SCALE).uniform(
            cfg.outlier_scale[0], cfg.outlier_scale[1], size=chans.size)
        X[:, chans] *= scales[None, :]
    elif cfg.x_model == "laplace":
        X = rx.laplace(0.0, 1.0, size=(M, K))
        if M > 0:
            base_max = np.max(np.abs(X[:, chans]))
            c = 1.0
            for _ in range(6):  # fixed point: c * base_max / median|X_scaled| -> target ratio
                Xs = X.copy()
                Xs[:, chans] *= c
                ratio = np.max(np.abs(Xs)) / np.median(np.abs(Xs))
                if abs(ratio / cfg.max_median_ratio - 1.0) < 1e-3:
                    break
                c = cfg.max_median_ratio * np.median(np.abs(Xs)) / base_max
            X[:, chans] *= c
    else:
        raise ValueError(cfg.x_model)

    W = make_rng(seed, cid, TAG_W).standard_normal((K, N)) / np.sqrt(K)
    if cfg.spike_rank > 0:
        rs = make_rng(seed, cid, TAG_SPIKE)
        qu, _ = np.linalg.qr(rs.standard_normal((K, cfg.spike_rank)))
        qv, _ = np.linalg.qr(rs.standard_normal((N, cfg.spike_rank)))
        W += cfg.spike_norm * (qu @ qv.T)

    bias = make_bias(cid, N, seed) if with_bias else None
    return dict(X=f64_to_bf16_bits(X), W=f64_to_bf16_bits(W), bias=bias,
                outlier_channels=chans, cfg=cfg, M=M, K=K, N=N)


def make_bias(cid: int, N: int, seed: int = 0) -> np.ndarray:
    """The seeded bias of a linear workload: N(0, 0.1^2) per output column, as bf16 bits (the
    same values ``make_linear(..., with_bias=True)`` returns)."""
    return f64_to_bf16_bits(make_rng(seed, cid, TAG_BIAS).normal(0.0, 0.1, size=N))


def make_kv(seed: int = 0, tokens: Optional[int] = None, heads: Optional[int] = None,
            dim: Optional[int] = None) -> dict:
    """Return {K, V} as bf16 bit patterns of shape [tokens, heads, dim]."""
    cfg = KV_CONFIG
    T = cfg.tokens if tokens is None else tokens
    H = cfg.heads if heads is None else heads
    D = cfg.dim if dim is None else dim
    C = H * D
    s = cfg.log_sigma
    mu = np.exp(s * s / 2.0)
    sd = np.sqrt((np.exp(s * s) - 1.0) * np.exp(s * s))
    zs = make_rng(seed, cfg.cid, TAG_CHANNEL_SIGMA).standard_normal(2 * C)
    out = {}
    for i, (name, tag) in enumerate((("K", TAG_K), ("V", TAG_V))):
        sigma_c = np.exp(cfg.channel_log_std * zs[i * C:(i + 1) * C])
        g = make_rng(seed, cfg.cid, tag).standard_normal((T, C))
        x = sigma_c[None, :] * (np.exp(s * g) - mu) / sd
        out[name] = f64_to_bf16_bits(x).reshape(T, H, D)
    out.update(tokens=T, heads=H, dim=D, cfg=cfg)
    return out
