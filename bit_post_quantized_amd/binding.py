"""ctypes binding of libsvdq (the C ABI in include/svdq.h), with the same function names.

Argument marshalling only: every function takes device tensors, passes their data pointers,
sizes and the current HIP stream to the library, and raises ``SvdqError`` on a nonzero status.
All computation happens in the library's kernels; there is no fallback path. PyTorch provides
device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsvdq.so")

SVDQ_OK, SVDQ_EINVAL, SVDQ_ESHAPE, SVDQ_EALIGN, SVDQ_EHIP = range(5)
SVDQ_OUT_BF16, SVDQ_OUT_FP32 = 0, 1

_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    "svdq_abi_version": ([], _I),
    "svdq_status_str": ([_I], ctypes.c_char_p),
    "svdq_last_error": ([], ctypes.c_char_p),
    "svdq_pack_weights": ([_P, _I, _I, _P, _P, _P], _I),
    "svdq_pack_lowrank": ([_P, _I, _I, _P, _P], _I),
    "svdq_pack_lowrank_up": ([_P, _I, _I, _P, _P], _I),
    "svdq_quantize_act": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "svdq_w4a4_gemm": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "svdq_w4a4_partials": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "svdq_e3m2_bytes": ([_I, _I], ctypes.c_size_t),
    "svdq_pack_weights_e3m2": ([_P, _I, _I, _P, _P, _P], _I),
    "svdq_quantize_act_e3m2": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "svdq_w4a4_gemm_e3m2": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "svdq_w4a4_partials_e3m2": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "svdq_quantize_act_a8": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "svdq_w4a8_gemm": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "svdq_w4a8_partials": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "kv_int8_workspace_bytes": ([_I, _I], ctypes.c_size_t),
    "kv_int8_quant": ([_P, _I, _I, _P, _P, _P, _P, _P], _I),
    "kv_int8_quant_pair": ([_P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "kv_int8_quant_pair_noalloc": ([_P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P], _I),
    "kv_int8_dequant": ([_P, _P, _P, _I, _I, _P, _P], _I),
    "kv_int8_attention_workspace_bytes": ([_I, _I, _I, _I], ctypes.c_size_t),
    "kv_int8_attention": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                           _P], _I),
}
EXPORTED = tuple(_SIGNATURES)


class SvdqError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (build it with ``python -m bit_post_quantized_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libsvdq.so not found at {path}; build it first "
                           "(python -m bit_post_quantized_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = lib
    return lib


_BF16, _F16, _F32, _U8, _I8, _I32 = (torch.bfloat16, torch.float16, torch.float32, torch.uint8,
                                     torch.int8, torch.int32)


class _Args:
    """Checks one call's tensors before their pointers go to the library: each must be a
    contiguous device tensor of the layout's dtype, on the same device as the others, holding
    at least the bytes the call reads or writes through it. The library cannot see buffer
    sizes or dtypes, so a short buffer would otherwise be read or written past its end and a
    wrong dtype read as other bits. None passes through as NULL, which the library rejects
    where the argument is required. Workspaces are raw bytes of any dtype."""

    def __init__(self, fn: str):
        self.fn = fn
        self.device: Optional[torch.device] = None

    def __call__(self, t: Optional[torch.Tensor], need: int, name: str,
                 dtype: Optional[torch.dtype] = None, shape: Optional[tuple] = None):
        if t is None:
            return None
        if not t.is_cuda:
            raise ValueError(f"{self.fn}: {name} must be a device tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{self.fn}: {name} must be {dtype} (got {t.dtype})")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.fn}: {name} must have shape {tuple(shape)} "
                             f"(got {tuple(t.shape)})")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous")
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            raise ValueError(f"{self.fn}: {name} is on {t.device}, "
                             f"other arguments on {self.device}")
        have = t.numel() * t.element_size()
        if have < need:
            raise ValueError(f"{self.fn}: {name} holds {have} bytes, the call needs {need}")
        return t.data_ptr()

    def stream(self, stream) -> Optional[int]:
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _out_dtype(fn: str, Y: torch.Tensor) -> int:
    if Y.dtype == torch.float32:
        return SVDQ_OUT_FP32
    if Y.dtype == torch.bfloat16:
        return SVDQ_OUT_BF16
    raise ValueError(f"{fn}: Y must be bfloat16 or float32 (got {Y.dtype})")


def _e3m2_bytes(rows: int, K: int) -> int:
    return load().svdq_e3m2_bytes(rows, K) if rows > 0 else 0


def _check(fn: str, status: int) -> None:
    if status != SVDQ_OK:
        lib = load()
        raise SvdqError(fn, status, lib.svdq_last_error().decode() or
                        lib.svdq_status_str(status).decode())


def svdq_abi_version() -> int:
    return load().svdq_abi_version()


def svdq_pack_weights(R: torch.Tensor, wq: torch.Tensor, w_scales: torch.Tensor,
                      stream=None) -> None:
    """R fp32 [K, N] -> wq uint8 [N, K/2], w_scales fp16 [K/64, N]."""
    fn = "svdq_pack_weights"
    K, N = R.shape
    a = _Args(fn)
    args = (a(R, 4 * K * N, "R", _F32), K, N, a(wq, N * (K // 2), "wq", _U8),
            a(w_scales, 2 * (K // 64) * N, "w_scales", _F16))
    _check(fn, load().svdq_pack_weights(*args, a.stream(stream)))


def svdq_pack_lowrank(L1: torch.Tensor, L1p: torch.Tensor, stream=None) -> None:
    """L1 bf16 [K, r] -> L1p bf16 [r, K], the activation pass's layout of the factor."""
    fn = "svdq_pack_lowrank"
    K, r = L1.shape
    a = _Args(fn)
    args = (a(L1, 2 * K * r, "L1", _BF16, (K, r)), K, r, a(L1p, 2 * r * K, "L1p", _BF16, (r, K)))
    _check(fn, load().svdq_pack_lowrank(*args, a.stream(stream)))


def svdq_pack_lowrank_up(L2: torch.Tensor, L2p: torch.Tensor, stream=None) -> None:
    """L2 bf16 [r, N] -> L2p bf16 [N, r], the GEMM epilogue's layout of the factor."""
    fn = "svdq_pack_lowrank_up"
    r, N = L2.shape
    a = _Args(fn)
    args = (a(L2, 2 * r * N, "L2", _BF16, (r, N)), r, N, a(L2p, 2 * N * r, "L2p", _BF16, (N, r)))
    _check(fn, load().svdq_pack_lowrank_up(*args, a.stream(stream)))


def svdq_quantize_act(X: torch.Tensor, inv_lambda: torch.Tensor, L1p: Optional[torch.Tensor],
                      r: int, xq: torch.Tensor, x_scales: torch.Tensor,
                      T: Optional[torch.Tensor], stream=None) -> None:
    """X bf16 [M, K], inv_lambda fp32 [K], L1p bf16 [r, K] (from svdq_pack_lowrank) ->
    xq uint8 [M, K/2], x_scales fp16 [M, K/64], T fp32 [M, r]."""
    _quantize_act("svdq_quantize_act", X, inv_lambda, L1p, r, xq, "xq",
                  X.shape[0] * (X.shape[1] // 2), x_scales, T, stream)


def _quantize_act(fn, X, inv_lambda, L1p, r, codes, code_name, code_bytes, x_scales, T,
                  stream) -> None:
    M, K = X.shape
    a = _Args(fn)
    args = (a(X, 2 * M * K, "X", _BF16, (M, K)), a(inv_lambda, 4 * K, "inv_lambda", _F32, (K,)),
            a(L1p, 2 * r * K, "L1p", _BF16, (r, K)), M, K, r,
            a(codes, code_bytes, code_name, _I8 if code_name == "xq8" else _U8),
            a(x_scales, 2 * (K // 64) * M, "x_scales", _F16, (M, K // 64)),
            a(T, 4 * M * r, "T", _F32, (M, r)))
    _check(fn, getattr(load(), fn)(*args, a.stream(stream)))


def _gemm(fn, xq, x_name, x_bytes, x_scales, T, wq, w_name, w_bytes, w_scales, L2p, bias, M, N,
          K, r, Y, stream) -> None:
    out = _out_dtype(fn, Y)
    a = _Args(fn)
    G = K // 64
    args = (a(xq, x_bytes, x_name, _I8 if x_name == "xq8" else _U8),
            a(x_scales, 2 * G * M, "x_scales", _F16, (M, G)), a(T, 4 * M * r, "T", _F32, (M, r)),
            a(wq, w_bytes, w_name, _U8), a(w_scales, 2 * G * N, "w_scales", _F16, (G, N)),
            a(L2p, 2 * N * r, "L2p", _BF16, (N, r)), a(bias, 2 * N, "bias", _BF16, (N,)),
            M, N, K, r, a(Y, Y.element_size() * M * N, "Y", None, (M, N)), out)
    _check(fn, getattr(load(), fn)(*args, a.stream(stream)))


def _partials(fn, xq, x_name, x_bytes, wq, w_name, w_bytes, M, N, K, P, stream) -> None:
    a = _Args(fn)
    args = (a(xq, x_bytes, x_name, _I8 if x_name == "xq8" else _U8),
            a(wq, w_bytes, w_name, _U8), M, N, K,
            a(P, 4 * (K // 64) * M * N, "P", _I32, (K // 64, M, N)))
    _check(fn, getattr(load(), fn)(*args, a.stream(stream)))


def svdq_w4a4_gemm(xq: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                   wq: torch.Tensor, w_scales: torch.Tensor, L2p: Optional[torch.Tensor],
                   bias: Optional[torch.Tensor], r: int, Y: torch.Tensor, stream=None) -> None:
    """Y [M, N] (bf16 or fp32, chosen by Y's dtype) of the fused W4A4 + low-rank GEMM."""
    M, half_k = xq.shape
    N = wq.shape[0]
    _gemm("svdq_w4a4_gemm", xq, "xq", M * half_k, x_scales, T, wq, "wq", N * half_k, w_scales,
          L2p, bias, M, N, 2 * half_k, r, Y, stream)


def svdq_w4a4_partials(xq: torch.Tensor, wq: torch.Tensor, P: torch.Tensor,
                       stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the GEMM's inner loop."""
    M, half_k = xq.shape
    N = wq.shape[0]
    _partials("svdq_w4a4_partials", xq, "xq", M * half_k, wq, "wq", N * half_k, M, N,
              2 * half_k, P, stream)


def svdq_e3m2_bytes(rows: int, K: int) -> int:
    """Bytes of the tiled BF6 code container of a [rows, K] code matrix."""
    return load().svdq_e3m2_bytes(rows, K)


def svdq_pack_weights_e3m2(R: torch.Tensor, wq6: torch.Tensor, w_scales: torch.Tensor,
                           stream=None) -> None:
    """R fp32 [K, N] -> wq6 (tiled BF6 container, svdq_e3m2_bytes(N, K) bytes), w_scales."""
    fn = "svdq_pack_weights_e3m2"
    K, N = R.shape
    a = _Args(fn)
    args = (a(R, 4 * K * N, "R", _F32), K, N, a(wq6, _e3m2_bytes(N, K), "wq6", _U8),
            a(w_scales, 2 * (K // 64) * N, "w_scales", _F16))
    _check(fn, load().svdq_pack_weights_e3m2(*args, a.stream(stream)))


def svdq_quantize_act_e3m2(X: torch.Tensor, inv_lambda: torch.Tensor,
                           L1p: Optional[torch.Tensor], r: int, xq6: torch.Tensor,
                           x_scales: torch.Tensor, T: Optional[torch.Tensor],
                           stream=None) -> None:
    """As svdq_quantize_act with the codes written to xq6, the tiled BF6 container of M rows."""
    _quantize_act("svdq_quantize_act_e3m2", X, inv_lambda, L1p, r, xq6, "xq6",
                  _e3m2_bytes(X.shape[0], X.shape[1]), x_scales, T, stream)


def svdq_w4a4_gemm_e3m2(xq6: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                        wq6: torch.Tensor, w_scales: torch.Tensor, L2p: Optional[torch.Tensor],
                        bias: Optional[torch.Tensor], r: int, Y: torch.Tensor,
                        stream=None) -> None:
    """As svdq_w4a4_gemm, reading the BF6 containers (M, N from Y [M, N], K from
    w_scales [K/64, N]; every other tensor's shape is checked against them)."""
    M, N = Y.shape
    G = w_scales.shape[0]
    K = 64 * G
    _gemm("svdq_w4a4_gemm_e3m2", xq6, "xq6", _e3m2_bytes(M, K), x_scales, T, wq6, "wq6",
          _e3m2_bytes(N, K), w_scales, L2p, bias, M, N, K, r, Y, stream)


def svdq_w4a4_partials_e3m2(xq6: torch.Tensor, wq6: torch.Tensor, M: int, N: int, K: int,
                            P: torch.Tensor, stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the BF6 GEMM's inner loop."""
    _partials("svdq_w4a4_partials_e3m2", xq6, "xq6", _e3m2_bytes(M, K), wq6, "wq6",
              _e3m2_bytes(N, K), M, N, K, P, stream)


def kv_int8_workspace_bytes(tokens: int, channels: int) -> int:
    return load().kv_int8_workspace_bytes(tokens, channels)


def _kv_shape(t: torch.Tensor):
    tokens = t.shape[0]
    channels = 1
    for d in t.shape[1:]:
        channels *= d
    return tokens, channels


def kv_int8_quant(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
                  workspace: Optional[torch.Tensor], stream=None) -> None:
    """x bf16 [tokens, ...] viewed as [tokens, channels] -> q uint8, scale fp32, zero uint8."""
    fn = "kv_int8_quant"
    tokens, channels = _kv_shape(x)
    a = _Args(fn)
    args = (a(x, 2 * tokens * channels, "x", _BF16), tokens, channels,
            a(q, tokens * channels, "q", _U8), a(scale, 4 * channels, "scale", _F32),
            a(zero, channels, "zero", _U8),
            a(workspace, kv_int8_workspace_bytes(tokens, channels) if tokens else 0, "workspace"))
    _check(fn, load().kv_int8_quant(*args, a.stream(stream)))


def kv_int8_quant_pair(k: torch.Tensor, v: torch.Tensor, qk: torch.Tensor, sk: torch.Tensor,
                       zk: torch.Tensor, qv: torch.Tensor, sv: torch.Tensor, zv: torch.Tensor,
                       workspace: Optional[torch.Tensor], stream=None) -> None:
    """kv_int8_quant of K and V (bf16, one shape [tokens, ...]) in one launch."""
    fn = "kv_int8_quant_pair"
    tokens, channels = _kv_shape(k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"{fn}: v must have the shape of k {tuple(k.shape)}, got {tuple(v.shape)}")
    a = _Args(fn)
    n = tokens * channels
    args = (a(k, 2 * n, "k", _BF16), a(v, 2 * n, "v", _BF16), tokens, channels,
            a(qk, n, "qk", _U8), a(sk, 4 * channels, "sk", _F32), a(zk, channels, "zk", _U8),
            a(qv, n, "qv", _U8), a(sv, 4 * channels, "sv", _F32), a(zv, channels, "zv", _U8),
            a(workspace, kv_int8_workspace_bytes(tokens, channels) if tokens else 0, "workspace"))
    _check(fn, load().kv_int8_quant_pair(*args, a.stream(stream)))


def kv_int8_quant_pair_noalloc(k: torch.Tensor, v: torch.Tensor, qk: torch.Tensor,
                               sk: torch.Tensor, zk: torch.Tensor, qv: torch.Tensor,
                               sv: torch.Tensor, zv: torch.Tensor, stream=None) -> None:
    """kv_int8_quant_pair on the library's own device scratch (no workspace, no allocation)."""
    fn = "kv_int8_quant_pair_noalloc"
    tokens, channels = _kv_shape(k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"{fn}: v must have the shape of k {tuple(k.shape)}, got {tuple(v.shape)}")
    a = _Args(fn)
    n = tokens * channels
    args = (a(k, 2 * n, "k", _BF16), a(v, 2 * n, "v", _BF16), tokens, channels,
            a(qk, n, "qk", _U8), a(sk, 4 * channels, "sk", _F32), a(zk, channels, "zk", _U8),
            a(qv, n, "qv", _U8), a(sv, 4 * channels, "sv", _F32), a(zv, channels, "zv", _U8))
    _check(fn, load().kv_int8_quant_pair_noalloc(*args, a.stream(stream)))


def kv_int8_dequant(q: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
                    x_out: torch.Tensor, stream=None) -> None:
    """q uint8 [tokens, ...] with its per-channel scale and zero -> x_out bf16, same shape."""
    fn = "kv_int8_dequant"
    tokens, channels = _kv_shape(q)
    a = _Args(fn)
    args = (a(q, tokens * channels, "q", _U8), a(scale, 4 * channels, "scale", _F32),
            a(zero, channels, "zero", _U8), tokens, channels,
            a(x_out, 2 * tokens * channels, "x_out", _BF16))
    _check(fn, load().kv_int8_dequant(*args, a.stream(stream)))


def svdq_quantize_act_a8(X: torch.Tensor, inv_lambda: torch.Tensor, L1p: Optional[torch.Tensor],
                         r: int, xq8: torch.Tensor, x_scales: torch.Tensor,
                         T: Optional[torch.Tensor], stream=None) -> None:
    """W4A8 activation pass: X bf16 [M, K] -> xq8 int8 [M, K], x_scales fp16 [M, K/64],
    T fp32 [M, r]."""
    _quantize_act("svdq_quantize_act_a8", X, inv_lambda, L1p, r, xq8, "xq8",
                  X.shape[0] * X.shape[1], x_scales, T, stream)


def svdq_w4a8_gemm(xq8: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                   wq: torch.Tensor, w_scales: torch.Tensor, L2p: Optional[torch.Tensor],
                   bias: Optional[torch.Tensor], r: int, Y: torch.Tensor, stream=None) -> None:
    """Y [M, N] of the W4A8 GEMM: int8 activation codes xq8 [M, K], INT4 nibbles wq [N, K/2]."""
    M, K = xq8.shape
    N = wq.shape[0]
    _gemm("svdq_w4a8_gemm", xq8, "xq8", M * K, x_scales, T, wq, "wq", N * (K // 2), w_scales,
          L2p, bias, M, N, K, r, Y, stream)


def svdq_w4a8_partials(xq8: torch.Tensor, wq: torch.Tensor, P: torch.Tensor,
                       stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the W4A8 GEMM's inner loop."""
    M, K = xq8.shape
    N = wq.shape[0]
    _partials("svdq_w4a8_partials", xq8, "xq8", M * K, wq, "wq", N * (K // 2), M, N, K, P,
              stream)


def kv_int8_attention_workspace_bytes(nq: int, tokens: int, heads: int, dim: int) -> int:
    return load().kv_int8_attention_workspace_bytes(nq, tokens, heads, dim)


def kv_int8_attention(q: torch.Tensor, k_codes: torch.Tensor, k_scale: torch.Tensor,
                      k_zero: torch.Tensor, v_codes: torch.Tensor, v_scale: torch.Tensor,
                      v_zero: torch.Tensor, sm_scale: float, out: torch.Tensor,
                      workspace: torch.Tensor, stream=None) -> None:
    """Decode attention over the INT8 cache: q bf16 [nq, heads, dim], codes uint8
    [tokens, heads * dim], per-channel scale / zero -> out bf16 [nq, heads, dim]."""
    fn = "kv_int8_attention"
    nq, heads, dim = q.shape
    tokens = k_codes.shape[0]
    C = heads * dim
    ws = kv_int8_attention_workspace_bytes(nq, tokens, heads, dim) if nq and tokens else 0
    a = _Args(fn)
    args = (a(q, 2 * nq * C, "q", _BF16), a(k_codes, tokens * C, "k_codes", _U8),
            a(k_scale, 4 * C, "k_scale", _F32), a(k_zero, C, "k_zero", _U8),
            a(v_codes, tokens * C, "v_codes", _U8), a(v_scale, 4 * C, "v_scale", _F32),
            a(v_zero, C, "v_zero", _U8), nq, tokens, heads, dim, float(sm_scale),
            a(out, 2 * nq * C, "out", _BF16), a(workspace, ws, "workspace"))
    _check(fn, load().kv_int8_attention(*args, a.stream(stream)))
