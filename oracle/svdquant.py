"""Oracle of the SVDQuant linear layer: Y ~ Q4(X diag(lam)^-1) Q4(R) + (X diag(lam)^-1 L1) L2.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__`` for the page short names cited below).

Layout convention: X is [M, K] (tokens x input channels), W is [K, N], Y = X W.  Groups are 64
consecutive input channels (k); G = K / 64.

Method, as the pages describe it (SVDQ "technical principles"; FLUX4 2.2 "three steps";
DCMP "SVDQuant" section):
  1. smoothing moves activation outliers into the weights:  X^ = X diag(lam)^-1, W^ = diag(lam) W;
  2. an SVD of W^ keeps the top-r singular triplets as a 16-bit low-rank branch L1 L2;
  3. the residual R = W^ - L1 L2 is quantized to 4 bits (the Eckart-Young-Mirsky theorem says
     removing the dominant singular values shrinks the residual's magnitude);
  4. activations are quantized dynamically at run time (FLUX4 3.1 "dynamic activation
     quantization"), with the symmetric rule of W4A8 3.1:
        scale = max|v| / (2^(b-1) - 1),  q = clamp(round(v / scale), -2^(b-1), 2^(b-1) - 1);
  5. Y = sum over groups of s_x s_w (integer dot products) + (X^ L1) L2 (+ bias).

Readings where the pages are silent (each listed with its reason in the design notes):
  * lam_k = max_m|X_mk|^alpha / max_n|W_kn|^(1-alpha) (SmoothQuant's rule; SmoothQuant is named on
    DCMP), lam_k = 1 when either max is 0; lam is stored as fp32 and the kernels get
    inv_lam = fl32(1 / lam32); W^ = lam32 * W in fp64.
  * L1 = U_r diag(S_r), L2 = V_r^T, both rounded to bf16; R = W^ - L1b L2b (against the rounded
    factors, so the 16-bit branch's rounding is absorbed by the residual), stored as fp32.
  * b = 4, groups of 64 along k for both X (per row) and R (per output column); the scale is
    s = fp16(fl32(amax / 7)) and codes are computed with the stored fp16 scale:
    q = clamp(rne(fl32(v / s)), -8, 7); s = 0 gives all-zero codes.
  * two codes per byte, even k in the low nibble, two's complement.
  * the low-rank product T = X^ L1b and the output are evaluated in fp64 here.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16, round_bf16, round_fp16

GROUP = 64
QMIN, QMAX = -8, 7


# --------------------------------------------------------------------------- weight preparation
def smoothing_factors(X: np.ndarray, W: np.ndarray, alpha: float):
    """Per-input-channel smoothing factor (SVDQ "technical principles": smoothing migrates
    activation outliers into the weights).

    X [M, K] and W [K, N] are float64. Returns (lam32, inv_lam32), both float32 [K].
    """
    a = np.max(np.abs(X), axis=0) if X.shape[0] else np.zeros(X.shape[1])
    w = np.max(np.abs(W), axis=1)
    lam = np.ones(X.shape[1], dtype=np.float64)
    ok = (a > 0) & (w > 0)
    lam[ok] = a[ok] ** alpha / w[ok] ** (1.0 - alpha)
    lam32 = lam.astype(np.float32)
    inv32 = np.float32(1.0) / lam32
    return lam32, inv32


def low_rank_split(W_hat: np.ndarray, rank: int) -> dict:
    """Truncated SVD of the smoothed weight (FLUX4 2.2, SVDQ "technical principles").

    Returns the fp64 factors (L1 = U_r S_r, L2 = V_r^T), their bf16 roundings, the fp64
    residual R = W^ - L1b L2b, R32 = fl32(R) and all singular values of W^.
    """
    K, N = W_hat.shape
    U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
    L1 = U[:, :rank] * S[None, :rank]
    L2 = Vt[:rank, :]
    L1b = round_bf16(L1)
    L2b = round_bf16(L2)
    R = W_hat - L1b @ L2b if rank > 0 else W_hat.copy()
    return dict(L1=L1, L2=L2, L1b=L1b, L2b=L2b, R=R, R32=R.astype(np.float32), S=S)


def prepare_weights(X_bits, W_bits, alpha: float, rank: int) -> dict:
    """Offline preparation: smoothing factors from the calibration activations, the low-rank
    split of the smoothed weight and the fp32 residual that gets quantized."""
    X = decode_bf16(X_bits)
    W = decode_bf16(W_bits)
    lam32, inv32 = smoothing_factors(X, W, alpha)
    W_hat = lam32.astype(np.float64)[:, None] * W
    out = low_rank_split(W_hat, rank)
    out.update(lam32=lam32, inv_lambda=inv32, W_hat=W_hat)
    return out


def attach_lora(L1b, L2b, lam32, A, B, scale: float = 1.0):
    """A low-rank adapter joins the 16-bit branch; the 4-bit residual is not re-quantized
    (SVDQ "feature list": LoRA adapters integrate without re-quantization).

    The adapter changes the layer to W' = W + scale * A B with A [K, r_l], B [r_l, N].  In the
    smoothed frame W^' = diag(lam) W' = W^ + (diag(lam) A)(scale B), and since the branch runs on
    X^ = X diag(lam)^-1 it computes X^ (diag(lam) A)(scale B) = scale * X A B.  So the adapter is
    appended as extra rank: L1' = [L1b | bf16(lam32 * A)], L2' = [L2b ; bf16(scale * B)].
    Returns (L1', L2') as float64 arrays holding bf16 values.
    """
    A_hat = round_bf16(np.asarray(lam32, dtype=np.float64)[:, None] * np.asarray(A, dtype=np.float64))
    B_s = round_bf16(scale * np.asarray(B, dtype=np.float64))
    return (np.concatenate([np.asarray(L1b, dtype=np.float64), A_hat], axis=1),
            np.concatenate([np.asarray(L2b, dtype=np.float64), B_s], axis=0))


# --------------------------------------------------------------------------- 4-bit quantizer
def quantize_groups(V32: np.ndarray, bits: int = 4):
    """Symmetric b-bit quantization of each length-64 vector along the last axis
    (W4A8 3.1 "quantization process": scale from the max magnitude over 2^(b-1)-1, round,
    clamp to the b-bit range).  b = 4 for the W4A4 path; b = 8 for the activations of the
    W4A8 variant.

    V32: float32 [..., 64]. Returns (codes int8 [..., 64], scales float16 [...]).
    """
    qmax = 2 ** (bits - 1) - 1
    qmin = -(2 ** (bits - 1))
    V32 = np.asarray(V32, dtype=np.float32)
    assert V32.shape[-1] == GROUP
    amax = np.max(np.abs(V32), axis=-1)
    s16 = round_fp16(amax / np.float32(qmax))
    if np.any(np.isinf(s16)):
        raise ValueError(f"group max / {qmax} exceeds the fp16 range (outside the contract)")
    s32 = s16.astype(np.float32)
    zero = s32 == 0
    quot = V32 / np.where(zero, np.float32(1.0), s32)[..., None]
    q = np.clip(np.rint(quot), qmin, qmax).astype(np.int8)
    q[zero] = 0
    return q, s16


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, K] int codes in [-8, 7] -> [rows, K/2] bytes; even k in the low nibble."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``: [rows, K/2] bytes -> [rows, K] int8 codes."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo, hi = p & 0xF, p >> 4
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int16)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def pack_weights(R32: np.ndarray) -> dict:
    """Quantize the fp32 residual R [K, N] per (64-group of k, output column n).

    Returns wq uint8 [N, K/2] (k-contiguous per column), s_w float16 [G, N], codes int8 [N, K].
    """
    K, N = R32.shape
    G = K // GROUP
    per_col = np.ascontiguousarray(np.asarray(R32, dtype=np.float32).T).reshape(N, G, GROUP)
    q, s16 = quantize_groups(per_col)
    codes = q.reshape(N, K)
    return dict(wq=pack_nibbles(codes), s_w=np.ascontiguousarray(s16.T), codes=codes)


# --------------------------------------------------------------------------- BF6 container
# FLUX4 3.2: on newer GPUs the matrix units read a small floating-point format directly, which
# removes the 4-bit unpack step that INT4 needs on INT8 units (W4A8 2.2).  The format with that
# property on the target GPU is BF6 = E3M2 as defined by the OCP Microscaling (MX) format
# specification v1.0 [external]: sign bit 5, exponent bits 4..2 with bias 3, mantissa bits
# 1..0; exponent 0 encodes the subnormals 2^-2 * m / 4.  Every integer in [-8, 8] is exactly
# representable, so the method's INT4 codes travel in it unchanged: only the container differs.
E3M2_BIAS = 3


def e3m2_value(bits) -> np.ndarray:
    """Value (float64) of each 6-bit E3M2 pattern, from the format definition."""
    b = np.asarray(bits, dtype=np.int64) & 0x3F
    sign = np.where(b >> 5, -1.0, 1.0)
    e = (b >> 2) & 0x7
    m = (b & 0x3).astype(np.float64)
    normal = np.ldexp(1.0 + m / 4.0, (e - E3M2_BIAS).astype(np.int64))
    sub = np.ldexp(m / 4.0, 1 - E3M2_BIAS)
    return sign * np.where(e == 0, sub, normal)


def e3m2_encode_codes(codes) -> np.ndarray:
    """Exact E3M2 pattern (uint8, 6 significant bits) of each integer code; zero encodes as +0.

    Raises ValueError for an integer the format cannot hold exactly (|c| > 8 or c = 9, 11, ...).
    """
    c = np.asarray(codes, dtype=np.int64)
    a = np.abs(c)
    out = np.zeros(c.shape, dtype=np.uint8)
    nz = a > 0
    e = np.zeros(c.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    frac = np.zeros(c.shape, dtype=np.float64)
    frac[nz] = a[nz] / np.ldexp(1.0, e[nz]) - 1.0          # in [0, 1)
    m = np.rint(frac * 4.0).astype(np.int64)
    exact = (~nz) | ((e + E3M2_BIAS <= 7) & (m < 4) & (frac * 4.0 == m))
    if not np.all(exact):
        raise ValueError("code not exactly representable in E3M2")
    out[nz] = (((c[nz] < 0).astype(np.int64) << 5) | ((e[nz] + E3M2_BIAS) << 2) | m[nz]).astype(np.uint8)
    return out


def pack_e3m2(codes: np.ndarray) -> np.ndarray:
    """[rows, K] int codes -> [rows, 3K/4] bytes: the codes' E3M2 patterns in k order, 6 bits
    each, as one little-endian bit stream per row (code k holds stream bits 6k .. 6k+5)."""
    pat = e3m2_encode_codes(codes)
    rows, K = pat.shape
    bits = ((pat[..., None] >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8)  # [rows, K, 6]
    return np.packbits(bits.reshape(rows, 6 * K), axis=1, bitorder="little")


def unpack_e3m2(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of ``pack_e3m2``: [rows, 3K/4] bytes -> [rows, K] int codes (values must be
    integers, as they are for every packed code)."""
    p = np.asarray(packed, dtype=np.uint8)
    bits = np.unpackbits(p, axis=1, bitorder="little")[:, : 6 * K].reshape(p.shape[0], K, 6)
    pat = (bits.astype(np.int64) << np.arange(6)).sum(axis=2)
    v = e3m2_value(pat)
    if not np.all(v == np.rint(v)):
        raise ValueError("packed value is not an integer code")
    return v.astype(np.int8)


E3M2_BLOCK_ROWS = 32       # rows per block of the tiled container
E3M2_SLOT_CODES = 32       # codes per slot (24 bytes)


def pack_e3m2_tiled(codes: np.ndarray) -> np.ndarray:
    """[R, K] int codes -> the tiled BF6 container, uint8 [ceil(R/32), K/64, 64, 24].

    Block b, group g, slot s holds the 32 codes of row 32 b + (s mod 32) at
    k = 64 g + 32 (s div 32) + i, i = 0..31, as the little-endian 6-bit stream of
    ``pack_e3m2`` (24 bytes).  Rows past R are zero codes.  (The order of slots within a block
    is the lane order of the 32 x 32 x 64 FP6 matrix-multiply operand.)
    """
    c = np.asarray(codes, dtype=np.int64)
    R, K = c.shape
    nb = -(-R // E3M2_BLOCK_ROWS)
    pad = np.zeros((nb * E3M2_BLOCK_ROWS, K), dtype=np.int64)
    pad[:R] = c
    G = K // GROUP
    # [block, row-in-block, group, half, 32 codes] -> [block, group, half, row-in-block, 32]
    v = pad.reshape(nb, E3M2_BLOCK_ROWS, G, 2, E3M2_SLOT_CODES).transpose(0, 2, 3, 1, 4)
    slots = pack_e3m2(v.reshape(-1, E3M2_SLOT_CODES))          # [n_slots, 24]
    return slots.reshape(nb, G, 2 * E3M2_BLOCK_ROWS, 24)


def unpack_e3m2_tiled(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of ``pack_e3m2_tiled``: the container (any shape of the same bytes) -> [R, K]."""
    G = K // GROUP
    nb = -(-R // E3M2_BLOCK_ROWS)
    b = np.asarray(buf, dtype=np.uint8).reshape(nb * G * 2 * E3M2_BLOCK_ROWS, 24)
    v = unpack_e3m2(b, E3M2_SLOT_CODES).reshape(nb, G, 2, E3M2_BLOCK_ROWS, E3M2_SLOT_CODES)
    return v.transpose(0, 3, 1, 2, 4).reshape(nb * E3M2_BLOCK_ROWS, K)[:R]


# --------------------------------------------------------------------------- activations
def smooth_activations(X_bits, inv_lam32: np.ndarray) -> np.ndarray:
    """X^ = fl32(fl32(X) * inv_lam): the smoothing divide as one fp32 multiply by the stored
    reciprocal."""
    X32 = decode_bf16(X_bits).astype(np.float32)
    return X32 * np.asarray(inv_lam32, dtype=np.float32)[None, :]


def quantize_act(X_bits, inv_lam32, L1b) -> dict:
    """Dynamic INT4 activation quantization per (token, 64-group) and the low-rank
    down-projection T = X^ L1b (fp64 of the fp32 X^)."""
    Xh = smooth_activations(X_bits, inv_lam32)
    M, K = Xh.shape
    G = K // GROUP
    q, s16 = quantize_groups(Xh.reshape(M, G, GROUP))
    codes = q.reshape(M, K)
    T = None
    if L1b is not None and np.asarray(L1b).shape[1] > 0:
        T = Xh.astype(np.float64) @ np.asarray(L1b, dtype=np.float64)
    return dict(xq=pack_nibbles(codes), s_x=s16, codes=codes, X_hat=Xh, T=T)


def quantize_act_a8(X_bits, inv_lam32, L1b) -> dict:
    """W4A8 variant of the activation pass (W4A8 1, 3.1: 8-bit activations, integers in
    [-128, 127], scale = max|v| / 127 per (token, 64-group)); smoothing and the low-rank
    down-projection are those of ``quantize_act``.  Returns codes int8 [M, K] (also the
    stored layout), s_x float16 [M, G], T."""
    Xh = smooth_activations(X_bits, inv_lam32)
    M, K = Xh.shape
    G = K // GROUP
    q, s16 = quantize_groups(Xh.reshape(M, G, GROUP), bits=8)
    codes = q.reshape(M, K)
    T = None
    if L1b is not None and np.asarray(L1b).shape[1] > 0:
        T = Xh.astype(np.float64) @ np.asarray(L1b, dtype=np.float64)
    return dict(xq8=codes.copy(), s_x=s16, codes=codes, X_hat=Xh, T=T)


# --------------------------------------------------------------------------- integer GEMM
def int_partials(cx: np.ndarray, cw: np.ndarray) -> np.ndarray:
    """P[g, m, n] = sum_{k in group g} cx[m, k] cw[n, k] (cx [M, K], cw [N, K] int codes).

    Evaluated with fp64 matrix products on integer-valued matrices: every product and partial
    sum is an integer of magnitude <= 64 * 128 * 8 (8-bit activation codes included), far below
    2^53, so the result is exact.
    """
    M, K = cx.shape
    N = cw.shape[0]
    G = K // GROUP
    P = np.empty((G, M, N), dtype=np.int32)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        P[g] = np.rint(cx[:, sl].astype(np.float64) @ cw[:, sl].astype(np.float64).T)
    return P


def int_partials_bruteforce(cx, cw):
    """Pure-Python triple loop of ``int_partials`` for tiny shapes."""
    M, K = len(cx), len(cx[0])
    N = len(cw)
    G = K // GROUP
    P = np.zeros((G, M, N), dtype=np.int64)
    for g in range(G):
        for m in range(M):
            for n in range(N):
                acc = 0
                for k in range(g * GROUP, (g + 1) * GROUP):
                    acc += int(cx[m][k]) * int(cw[n][k])
                P[g, m, n] = acc
    return P


def linear_output(cx, s_x, cw, s_w, T=None, L2b=None, bias_bits=None) -> np.ndarray:
    """Y[m, n] = sum_g s_x[m, g] s_w[g, n] P[g, m, n] + (T L2b)[m, n] + bias[n]   (fp64).

    The low-rank term is the 16-bit branch kept beside the 4-bit product (SVDQ "technical
    principles"); the bias is optional.
    """
    M, K = cx.shape
    N = cw.shape[0]
    G = K // GROUP
    Y = np.zeros((M, N), dtype=np.float64)
    sx = np.asarray(s_x, dtype=np.float64)
    sw = np.asarray(s_w, dtype=np.float64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        Pg = cx[:, sl].astype(np.float64) @ cw[:, sl].astype(np.float64).T
        Y += (sx[:, g:g + 1] * sw[g:g + 1, :]) * Pg
    if T is not None and L2b is not None and np.asarray(L2b).shape[0] > 0:
        Y += np.asarray(T, dtype=np.float64) @ np.asarray(L2b, dtype=np.float64)
    if bias_bits is not None:
        Y += decode_bf16(bias_bits)[None, :]
    return Y


def svdq_linear(X_bits, inv_lam32, L1b, L2b, packed_w: dict, bias_bits=None) -> dict:
    """Whole forward pass of one SVDQuant linear given prepared weights."""
    act = quantize_act(X_bits, inv_lam32, L1b)
    Y = linear_output(act["codes"], act["s_x"], packed_w["codes"], packed_w["s_w"],
                      act["T"], L2b, bias_bits)
    act["Y"] = Y
    return act
