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


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libsvdq takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libsvdq takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


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
    K, N = R.shape
    _check("svdq_pack_weights", load().svdq_pack_weights(
        _ptr(R), K, N, _ptr(wq), _ptr(w_scales), _stream(stream)))


def svdq_quantize_act(X: torch.Tensor, inv_lambda: torch.Tensor, L1: Optional[torch.Tensor],
                      r: int, xq: torch.Tensor, x_scales: torch.Tensor,
                      T: Optional[torch.Tensor], stream=None) -> None:
    """X bf16 [M, K], inv_lambda fp32 [K], L1 bf16 [r, K] (K-contiguous) ->
    xq uint8 [M, K/2], x_scales fp16 [K/64, M], T fp32 [M, r]."""
    M, K = X.shape
    _check("svdq_quantize_act", load().svdq_quantize_act(
        _ptr(X), _ptr(inv_lambda), _ptr(L1), M, K, r, _ptr(xq), _ptr(x_scales), _ptr(T),
        _stream(stream)))


def svdq_w4a4_gemm(xq: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                   wq: torch.Tensor, w_scales: torch.Tensor, L2: Optional[torch.Tensor],
                   bias: Optional[torch.Tensor], r: int, Y: torch.Tensor, stream=None) -> None:
    """Y [M, N] (bf16 or fp32, chosen by Y's dtype) of the fused W4A4 + low-rank GEMM."""
    M, half_k = xq.shape
    N = wq.shape[0]
    out = SVDQ_OUT_FP32 if Y.dtype == torch.float32 else SVDQ_OUT_BF16
    _check("svdq_w4a4_gemm", load().svdq_w4a4_gemm(
        _ptr(xq), _ptr(x_scales), _ptr(T), _ptr(wq), _ptr(w_scales), _ptr(L2), _ptr(bias),
        M, N, 2 * half_k, r, _ptr(Y), out, _stream(stream)))


def svdq_w4a4_partials(xq: torch.Tensor, wq: torch.Tensor, P: torch.Tensor,
                       stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the GEMM's inner loop."""
    M, half_k = xq.shape
    N = wq.shape[0]
    _check("svdq_w4a4_partials", load().svdq_w4a4_partials(
        _ptr(xq), _ptr(wq), M, N, 2 * half_k, _ptr(P), _stream(stream)))


def svdq_e3m2_bytes(rows: int, K: int) -> int:
    """Bytes of the tiled BF6 code container of a [rows, K] code matrix."""
    return load().svdq_e3m2_bytes(rows, K)


def svdq_pack_weights_e3m2(R: torch.Tensor, wq6: torch.Tensor, w_scales: torch.Tensor,
                           stream=None) -> None:
    """R fp32 [K, N] -> wq6 (tiled BF6 container, svdq_e3m2_bytes(N, K) bytes), w_scales."""
    K, N = R.shape
    _check("svdq_pack_weights_e3m2", load().svdq_pack_weights_e3m2(
        _ptr(R), K, N, _ptr(wq6), _ptr(w_scales), _stream(stream)))


def svdq_quantize_act_e3m2(X: torch.Tensor, inv_lambda: torch.Tensor,
                           L1: Optional[torch.Tensor], r: int, xq6: torch.Tensor,
                           x_scales: torch.Tensor, T: Optional[torch.Tensor],
                           stream=None) -> None:
    """As svdq_quantize_act with the codes written to xq6, the tiled BF6 container of M rows."""
    M, K = X.shape
    _check("svdq_quantize_act_e3m2", load().svdq_quantize_act_e3m2(
        _ptr(X), _ptr(inv_lambda), _ptr(L1), M, K, r, _ptr(xq6), _ptr(x_scales), _ptr(T),
        _stream(stream)))


def svdq_w4a4_gemm_e3m2(xq6: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                        wq6: torch.Tensor, w_scales: torch.Tensor, L2: Optional[torch.Tensor],
                        bias: Optional[torch.Tensor], r: int, Y: torch.Tensor,
                        stream=None) -> None:
    """As svdq_w4a4_gemm, reading the BF6 containers (M, N, K from x_scales [K/64, M] and
    w_scales [K/64, N])."""
    G, M = x_scales.shape
    N = w_scales.shape[1]
    out = SVDQ_OUT_FP32 if Y.dtype == torch.float32 else SVDQ_OUT_BF16
    _check("svdq_w4a4_gemm_e3m2", load().svdq_w4a4_gemm_e3m2(
        _ptr(xq6), _ptr(x_scales), _ptr(T), _ptr(wq6), _ptr(w_scales), _ptr(L2), _ptr(bias),
        M, N, 64 * G, r, _ptr(Y), out, _stream(stream)))


def svdq_w4a4_partials_e3m2(xq6: torch.Tensor, wq6: torch.Tensor, M: int, N: int, K: int,
                            P: torch.Tensor, stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the BF6 GEMM's inner loop."""
    _check("svdq_w4a4_partials_e3m2", load().svdq_w4a4_partials_e3m2(
        _ptr(xq6), _ptr(wq6), M, N, K, _ptr(P), _stream(stream)))


def kv_int8_workspace_bytes(tokens: int, channels: int) -> int:
    return load().kv_int8_workspace_bytes(tokens, channels)


def kv_int8_quant(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
                  workspace: Optional[torch.Tensor], stream=None) -> None:
    """x bf16 [tokens, ...] viewed as [tokens, channels] -> q uint8, scale fp32, zero uint8."""
    tokens = x.shape[0]
    channels = x.numel() // tokens if tokens else int(torch.tensor(x.shape[1:]).prod())
    _check("kv_int8_quant", load().kv_int8_quant(
        _ptr(x), tokens, channels, _ptr(q), _ptr(scale), _ptr(zero), _ptr(workspace),
        _stream(stream)))


def kv_int8_dequant(q: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
                    x_out: torch.Tensor, stream=None) -> None:
    tokens = q.shape[0]
    channels = q.numel() // tokens if tokens else int(torch.tensor(q.shape[1:]).prod())
    _check("kv_int8_dequant", load().kv_int8_dequant(
        _ptr(q), _ptr(scale), _ptr(zero), tokens, channels, _ptr(x_out), _stream(stream)))


def svdq_quantize_act_a8(X: torch.Tensor, inv_lambda: torch.Tensor, L1: Optional[torch.Tensor],
                         r: int, xq8: torch.Tensor, x_scales: torch.Tensor,
                         T: Optional[torch.Tensor], stream=None) -> None:
    """W4A8 activation pass: X bf16 [M, K] -> xq8 int8 [M, K], x_scales fp16 [K/64, M],
    T fp32 [M, r]."""
    M, K = X.shape
    _check("svdq_quantize_act_a8", load().svdq_quantize_act_a8(
        _ptr(X), _ptr(inv_lambda), _ptr(L1), M, K, r, _ptr(xq8), _ptr(x_scales), _ptr(T),
        _stream(stream)))


def svdq_w4a8_gemm(xq8: torch.Tensor, x_scales: torch.Tensor, T: Optional[torch.Tensor],
                   wq: torch.Tensor, w_scales: torch.Tensor, L2: Optional[torch.Tensor],
                   bias: Optional[torch.Tensor], r: int, Y: torch.Tensor, stream=None) -> None:
    """Y [M, N] of the W4A8 GEMM: int8 activation codes xq8 [M, K], INT4 nibbles wq [N, K/2]."""
    M, K = xq8.shape
    N = wq.shape[0]
    out = SVDQ_OUT_FP32 if Y.dtype == torch.float32 else SVDQ_OUT_BF16
    _check("svdq_w4a8_gemm", load().svdq_w4a8_gemm(
        _ptr(xq8), _ptr(x_scales), _ptr(T), _ptr(wq), _ptr(w_scales), _ptr(L2), _ptr(bias),
        M, N, K, r, _ptr(Y), out, _stream(stream)))


def svdq_w4a8_partials(xq8: torch.Tensor, wq: torch.Tensor, P: torch.Tensor,
                       stream=None) -> None:
    """P int32 [K/64, M, N]: the exact group partials of the W4A8 GEMM's inner loop."""
    M, K = xq8.shape
    N = wq.shape[0]
    _check("svdq_w4a8_partials", load().svdq_w4a8_partials(
        _ptr(xq8), _ptr(wq), M, N, K, _ptr(P), _stream(stream)))


def kv_int8_attention_workspace_bytes(nq: int, tokens: int, heads: int, dim: int) -> int:
    return load().kv_int8_attention_workspace_bytes(nq, tokens, heads, dim)


def kv_int8_attention(q: torch.Tensor, k_codes: torch.Tensor, k_scale: torch.Tensor,
                      k_zero: torch.Tensor, v_codes: torch.Tensor, v_scale: torch.Tensor,
                      v_zero: torch.Tensor, sm_scale: float, out: torch.Tensor,
                      workspace: torch.Tensor, stream=None) -> None:
    """Decode attention over the INT8 cache: q bf16 [nq, heads, dim], codes uint8
    [tokens, heads * dim], per-channel scale / zero -> out bf16 [nq, heads, dim]."""
    nq, heads, dim = q.shape
    tokens = k_codes.shape[0]
    _check("kv_int8_attention", load().kv_int8_attention(
        _ptr(q), _ptr(k_codes), _ptr(k_scale), _ptr(k_zero), _ptr(v_codes), _ptr(v_scale),
        _ptr(v_zero), nq, tokens, heads, dim, float(sm_scale), _ptr(out), _ptr(workspace),
        _stream(stream)))
