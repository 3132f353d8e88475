/*
 * svdq.h — C ABI of the MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer and the INT8
 * KV-cache quantizer.
 *
 * Sources (web pages), cited below by short name:
 *   SVDQ  "SVDQuant是什么？一文让你看懂SVDQuant的技术原理、主要功能、应用场景" (zhuoshang.net)
 *   FLUX4 "AI图像生成4-bit量化技术解析与应用" (intelliparadigm.com)
 *   W4A8  "W4A8量化技术在边缘计算中的实践与优化" (mhpn.cn)
 *   VARC  "VAR-Compressor：在边缘GPU上实现80亿参数视觉自回归模型的高效量化部署" (zingnex.cn)
 *   DCMP  "DeepCompressor：MIT 团队开源的大模型与 Diffusion 模型压缩工具箱" (pomoai.com)
 *
 * The layer computes  Y = Q4(X diag(lam)^-1) Q4(R) + (X diag(lam)^-1 L1) L2 + bias  where the
 * weight W [K, N] was smoothed (W^ = diag(lam) W), split by a rank-r SVD into a 16-bit branch
 * L1 [K, r] L2 [r, N] and a residual R = W^ - L1 L2 that is quantized to 4 bits
 * (SVDQ "technical principles"; FLUX4 2.2).  G = K / 64 quantization groups along K.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or keeps them, holds no global state (apart from the device scratch of
 *     kv_int8_quant_pair_noalloc) and is safe to call from several threads.
 *   - Arrays are dense and row-major in the layout written next to each argument; fp16 and
 *     bf16 values are passed as their uint16 bit patterns.
 *   - Pointers marked "16B" must be 16-byte aligned.
 *   - Every call validates its arguments synchronously and, on error, returns a nonzero status
 *     and launches nothing (outputs untouched).  On success the work is enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream) and the call returns at once;
 *     faults inside a kernel surface at the caller's next synchronization.
 *   - Sizes of 0 rows (M = 0, tokens = 0) are valid and enqueue nothing.
 *   - Inputs that are NaN or Inf, or whose group max / 7 exceeds the fp16 range (65504), are
 *     outside the contract: the call succeeds but the codes and scales are unspecified.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 8

enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_EINVAL = 1, /* NULL pointer, negative or zero size where one is required */
  SVDQ_ESHAPE = 2, /* K % 64 != 0, r % 16 != 0 or r > 128, channels % 8 != 0, too large */
  SVDQ_EALIGN = 3, /* a "16B" pointer is not 16-byte aligned */
  SVDQ_EHIP = 4    /* the HIP runtime refused the launch (see svdq_last_error) */
};

enum svdq_out_dtype { SVDQ_OUT_BF16 = 0, SVDQ_OUT_FP32 = 1 };

/* SVDQ_ABI_VERSION of the built library. */
int svdq_abi_version(void);

/* Static text for a status code. */
const char* svdq_status_str(int status);

/* Text of the last error raised on the calling thread (empty if none). */
const char* svdq_last_error(void);

/*
 * svdq_pack_weights — quantize the fp32 residual R to symmetric INT4 per (64-group of k,
 * output column n) and pack two codes per byte (residual quantization: FLUX4 2.2; scale rule
 * W4A8 3.1 with b = 4).  For each (g, n):
 *     s = fp16(fl32(amax / 7)),  q = clamp(rne(fl32(R / s)), -8, 7),  q = 0 when s == 0.
 *   R         fp32 [K, N]                       16B
 *   wq        uint8 [N, K/2]; byte j of row n holds k = 2j (low nibble) and 2j+1 (high)  16B
 *   w_scales  fp16 [G, N]
 *   K % 64 == 0, K >= 64, N >= 1.  Offline (weight preparation), not on the timed path.
 */
int svdq_pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                      void* stream);

/*
 * svdq_pack_lowrank — relayout of the 16-bit branch's down-projection factor for the activation
 * pass (offline weight preparation, like svdq_pack_weights; SVDQ "technical principles": the
 * rank-r branch L1 L2 kept in 16 bits).  Values are copied, not rounded.
 *   L1    bf16 [K, r] (row-major: element (k, j) at L1[k * r + j])
 *   L1p   bf16 [r, K] (element (k, j) at L1p[j * K + k]: each rank's K values contiguous)
 *   K % 64 == 0, K >= 64, 16 <= r <= 128, r % 16 == 0.
 */
int svdq_pack_lowrank(const uint16_t* L1, int K, int r, uint16_t* L1p, void* stream);

/*
 * svdq_pack_lowrank_up — relayout of the 16-bit branch's up-projection factor for the GEMM
 * epilogue (offline weight preparation, like svdq_pack_lowrank; SVDQ "technical principles":
 * the rank-r branch L1 L2 kept in 16 bits).  Values are copied, not rounded.
 *   L2    bf16 [r, N] (row-major: element (j, n) at L2[j * N + n])
 *   L2p   bf16 [N, r] (element (j, n) at L2p[n * r + j]: each column's r values contiguous)
 *   16 <= r <= 128, r % 16 == 0, 1 <= N <= 2^24.
 */
int svdq_pack_lowrank_up(const uint16_t* L2, int r, int N, uint16_t* L2p, void* stream);

/*
 * svdq_quantize_act — one HBM pass over the activations: smoothing divide (a multiply by the
 * stored reciprocal inv_lambda), dynamic symmetric INT4 quantization per (token, 64-group)
 * (FLUX4 3.1 "dynamic activation quantization"; W4A8 3.1), and the low-rank down-projection
 * T = bf16(X^) L1 with fp32 accumulation (SVDQ "technical principles": 16-bit branch).
 *     X^ = fl32(X * inv_lambda);  s = fp16(fl32(amax / 7));  q = clamp(rne(fl32(X^ / s)), -8, 7)
 *   X           bf16 [M, K]                               16B
 *   inv_lambda  fp32 [K]                                  16B
 *   L1p         bf16 [r, K], the factor L1 [K, r] as written by svdq_pack_lowrank (16B); may be
 *               NULL when r == 0
 *   xq          uint8 [M, K/2], nibble order as wq        16B
 *   x_scales    fp16 [M, K/64] (row-major: token m's G scales contiguous)
 *   T           fp32 [M, r]; may be NULL when r == 0
 *   M >= 0, K % 64 == 0, K >= 64, 0 <= r <= 128, r % 16 == 0.
 */
int svdq_quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1p, int M,
                      int K, int r, uint8_t* xq, uint16_t* x_scales, float* T, void* stream);

/*
 * svdq_w4a4_gemm — the W4A4 group GEMM with the low-rank branch and bias fused into its
 * epilogue (SVDQ "Nunchaku" kernel fusion; DCMP "SVDQuant" section):
 *     Y[m, n] = sum_g s_x[m, g] s_w[g, n] P[g, m, n] + (bf16(T) L2)[m, n] + bias[n],
 *     P[g, m, n] = sum_{k in group g} qx[m, k] qw[n, k]   (exact int32).
 *   xq, x_scales, T   as written by svdq_quantize_act (T: 16B; may be NULL when r == 0)
 *   wq, w_scales      as written by svdq_pack_weights
 *   L2p         bf16 [N, r], the factor L2 [r, N] as written by svdq_pack_lowrank_up (16B);
 *               may be NULL when r == 0
 *   bias        bf16 [N] or NULL
 *   Y           [M, N], bf16 (out_dtype = SVDQ_OUT_BF16, round to nearest even) or fp32
 *               (SVDQ_OUT_FP32)                           16B
 *   M >= 0, 1 <= N <= 2^24, K % 64 == 0, 64 <= K <= 64 * 65535 (the packer's limit),
 *   0 <= r <= 128, r % 16 == 0.  The same limits hold for every GEMM entry point below.
 */
int svdq_w4a4_gemm(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                   const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2p,
                   const uint16_t* bias, int M, int N, int K, int r, void* Y, int out_dtype,
                   void* stream);

/*
 * svdq_w4a4_partials — test entry: the exact int32 group partials of the same device inner
 * loop as svdq_w4a4_gemm, P[g][m][n] = sum_{k in group g} qx[m, k] qw[n, k] (the integer dot
 * products of 4-bit codes that W4A8 2.2 and 4.2 run on the 8-bit units, here one per 64-group).
 *   P  int32 [G, M, N]
 */
int svdq_w4a4_partials(const uint8_t* xq, const uint8_t* wq, int M, int N, int K, int32_t* P,
                       void* stream);

/*
 * BF6 (E3M2) tiled container.  The *_e3m2 entry points compute exactly the same codes, scales,
 * T and Y as the entry points above; only the container of the codes differs.  Each code is
 * stored as its 6-bit BF6 pattern (OCP Microscaling format E3M2: sign bit 5, exponent bits 4..2
 * with bias 3, mantissa bits 1..0; every integer in [-8, 8] is exact).  A [R, K] code matrix
 * (R = M for activations, N for weights) is stored as ceil(R / 32) row blocks; block b holds,
 * for each 64-group g in order, 64 slots of 24 bytes; slot s carries the 32 codes of row
 * 32 b + (s mod 32) at k = 64 g + 32 (s div 32) + i, i = 0..31, as one little-endian 192-bit
 * stream (code i at bits 6i .. 6i+5).  Rows past R hold zero codes (the quantize/pack calls
 * write them).  The slot order is the lane order of the gfx950 32 x 32 x 64 FP6 matrix
 * operand, so the GEMM copies whole blocks (FLUX4 3.2: a small float format on the matrix
 * units avoids the 4-bit unpack).  Size: svdq_e3m2_bytes(R, K) bytes, 16-byte aligned.
 *
 * svdq_e3m2_bytes — ceil(rows / 32) * (K / 64) * 1536 (0 for rows <= 0 or K not a positive
 *   multiple of 64).
 * svdq_pack_weights_e3m2 — svdq_pack_weights writing wq6 (container of N rows) instead of wq.
 * svdq_quantize_act_e3m2 — svdq_quantize_act writing xq6 (container of M rows) instead of xq.
 * svdq_w4a4_gemm_e3m2 — svdq_w4a4_gemm reading xq6 / wq6 (same Y up to fp32 summation order).
 * svdq_w4a4_partials_e3m2 — test entry: the exact group partials of the same device inner loop
 *   as svdq_w4a4_gemm_e3m2, P int32 [G, M, N].
 * Arguments, shapes, alignment and error behaviour are otherwise those of the matching entry
 * point above.
 */
size_t svdq_e3m2_bytes(int rows, int K);
int svdq_pack_weights_e3m2(const float* R, int K, int N, uint8_t* wq6, uint16_t* w_scales,
                           void* stream);
int svdq_quantize_act_e3m2(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                           int M, int K, int r, uint8_t* xq6, uint16_t* x_scales, float* T,
                           void* stream);
int svdq_w4a4_gemm_e3m2(const uint8_t* xq6, const uint16_t* x_scales, const float* T,
                        const uint8_t* wq6, const uint16_t* w_scales, const uint16_t* L2p,
                        const uint16_t* bias, int M, int N, int K, int r, void* Y,
                        int out_dtype, void* stream);
int svdq_w4a4_partials_e3m2(const uint8_t* xq6, const uint8_t* wq6, int M, int N, int K,
                            int32_t* P, void* stream);

/*
 * W4A8 variant (W4A8 sections 1, 3.1, 2.2: 8-bit activations, 4-bit weights widened to 8 bits
 * on the INT8 units).  The activation codes are 8-bit, per (token, 64-group):
 *     s = fp16(fl32(amax / 127)),  q = clamp(rne(fl32(x^ / s)), -128, 127),  q = 0 when s == 0,
 * with the smoothing and the low-rank down-projection T of svdq_quantize_act; the weights are
 * those of svdq_pack_weights (INT4 nibbles), and
 *     Y[m, n] = sum_g s_x[m, g] s_w[g, n] P[g, m, n] + (bf16(T) L2)[m, n] + bias[n],
 *     P[g, m, n] = sum_{k in group g} q8x[m, k] qw[n, k]   (exact int32).
 * svdq_quantize_act_a8 — svdq_quantize_act writing xq8, int8 [M, K] (two's complement, one code
 *   per byte, 16B) instead of nibbles.
 * svdq_w4a8_gemm — svdq_w4a4_gemm reading xq8 instead of xq.
 * svdq_w4a8_partials — test entry: the exact group partials of the same device inner loop as
 *   svdq_w4a8_gemm, P int32 [G, M, N].
 * Arguments, shapes, alignment and error behaviour are otherwise those of the matching W4A4
 * entry point.
 */
int svdq_quantize_act_a8(const uint16_t* X, const float* inv_lambda, const uint16_t* L1, int M,
                         int K, int r, int8_t* xq8, uint16_t* x_scales, float* T, void* stream);
int svdq_w4a8_gemm(const int8_t* xq8, const uint16_t* x_scales, const float* T,
                   const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2p,
                   const uint16_t* bias, int M, int N, int K, int r, void* Y, int out_dtype,
                   void* stream);
int svdq_w4a8_partials(const int8_t* xq8, const uint8_t* wq, int M, int N, int K, int32_t* P,
                       void* stream);

/*
 * kv_int8_workspace_bytes — size of the caller-owned scratch that kv_int8_quant and
 * kv_int8_quant_pair need for the cross-token min/max reduction of their per-channel ranges
 * (VARC "INT8 KV cache quantization": statistics per channel over the cached tokens; 0 when
 * tokens == 0): the per-part partial ranges and tags of the single-pass schedule (two tensors'
 * worth, for the paired call), or the per-64-token-chunk partials of the three-pass schedule
 * for shapes the single pass does not take; the size covers every case of both calls.  Its
 * contents need no initialization and carry nothing between calls (a tag left by an earlier
 * call never matches a later one); calls that share one workspace must not overlap in time
 * (one stream, or one workspace per stream).
 */
size_t kv_int8_workspace_bytes(int tokens, int channels);

/*
 * kv_int8_quant — asymmetric per-channel INT8 quantization of a KV-cache tensor viewed as
 * x [tokens, channels] (channel = one (head, dim) pair; statistics over every token of the
 * call), VARC "INT8 KV cache quantization":
 *     lo = min(0, min_t x), hi = max(0, max_t x), s = fl32(fl32(hi - lo) / 255) (1 if 0),
 *     z = clamp(rne(fl32(-lo / s)), 0, 255),  q = clamp(rne(fl32(x / s)) + z, 0, 255).
 *   x          bf16 [tokens, channels]                    16B
 *   q          uint8 [tokens, channels]                   16B
 *   scale      fp32 [channels]    16B;   zero  uint8 [channels]    16B
 *   workspace  device scratch of kv_int8_workspace_bytes(tokens, channels) bytes    16B
 *   0 <= tokens <= 2097120 (65535 * 32), channels >= 8, channels % 8 == 0.
 */
int kv_int8_quant(const uint16_t* x, int tokens, int channels, uint8_t* q, float* scale,
                  uint8_t* zero, void* workspace, void* stream);

/*
 * kv_int8_quant_pair — kv_int8_quant of two tensors of one shape, a layer's K and V cache
 * (VARC "INT8 KV cache quantization": both caches are stored as per-channel INT8), in one
 * launch: the codes, scales and zeros are those of two kv_int8_quant calls, bit for bit.  The
 * single-pass schedule stores K's codes while it reads V, so the two tensors' traffic overlaps;
 * shapes the single pass does not take run two kv_int8_quant calls on the stream.
 *   k, v          bf16 [tokens, channels]                          16B
 *   qk, qv        uint8 [tokens, channels]                         16B
 *   sk, sv        fp32 [channels] (16B);  zk, zv  uint8 [channels] (16B)
 *   workspace     device scratch of kv_int8_workspace_bytes(tokens, channels) bytes   16B
 *   Limits and errors as kv_int8_quant.  No output may overlap an input or another output.
 */
int kv_int8_quant_pair(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                       uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv, uint8_t* zv,
                       void* workspace, void* stream);

/*
 * kv_int8_quant_pair_noalloc — kv_int8_quant_pair without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The scratch is a 16 MiB array in the
 * library's device code, which every device the library runs on holds until the process ends;
 * the call makes no hipMalloc, hipFree or other allocating call.  Same arguments (less
 * workspace), results and limits as kv_int8_quant_pair, and additionally
 * kv_int8_workspace_bytes(tokens, channels) <= 16 MiB (SVDQ_ESHAPE otherwise; e.g. 10240 tokens
 * x 4096 channels need 5 MiB).  The scratch carries nothing between calls, but all calls on one
 * device share it: calls that overlap in time on one device (several streams, or several host
 * threads) race and must be serialized by the caller.
 */
int kv_int8_quant_pair_noalloc(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                               uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv,
                               uint8_t* zv, void* stream);

/*
 * kv_int8_dequant — the inverse map of kv_int8_quant's affine code (VARC "INT8 KV cache
 * quantization": per-channel scale and non-centered zero point),
 *     x' = bf16(fl32((q - z) * s)) per element (round to nearest even).
 *   q      uint8 [tokens, channels]   16B;   x_out  bf16 [tokens, channels]   16B
 *   scale, zero as written by kv_int8_quant   16B
 *   0 <= tokens <= 2097120 (65535 * 32), channels >= 8, channels % 8 == 0.
 */
int kv_int8_dequant(const uint8_t* q, const float* scale, const uint8_t* zero, int tokens,
                    int channels, uint16_t* x_out, void* stream);

/*
 * kv_int8_attention — decode attention that reads the INT8 cache written by kv_int8_quant
 * (the consumer that turns the cache's memory saving into a bandwidth saving; VARC "INT8 KV
 * cache quantization").  For every query i and head h, over all tokens t:
 *     K'[t, c] = (k_codes[t, c] - k_zero[c]) k_scale[c],  V' likewise,  c = h dim + d,
 *     out[i, h, :] = softmax_t(sm_scale q[i, h, :] . K'[t, h, :]) V'[t, h, :]
 * evaluated in fp32 (scores, weights and the code-space sums) and rounded to bf16.
 *   q          bf16 [nq, heads, dim]                                   16B
 *   k_codes, v_codes   uint8 [tokens, heads dim] as written by kv_int8_quant   16B
 *   k_scale, k_zero    fp32 / uint8 [heads dim] (16B); v_scale, v_zero likewise
 *   out        bf16 [nq, heads, dim]
 *   workspace  device scratch of kv_int8_attention_workspace_bytes(nq, tokens, heads, dim)
 *              bytes (16B): one partial (max, sum, dim code-space sums) per query, head and
 *              256-token chunk; no initialization needed, fully rewritten by every call; calls
 *              that share one workspace must not overlap in time.
 *   nq >= 1, 1 <= tokens <= 2^20, heads >= 1, dim 64 or 128, sm_scale finite.
 */
size_t kv_int8_attention_workspace_bytes(int nq, int tokens, int heads, int dim);
int kv_int8_attention(const uint16_t* q, const uint8_t* k_codes, const float* k_scale,
                      const uint8_t* k_zero, const uint8_t* v_codes, const float* v_scale,
                      const uint8_t* v_zero, int nq, int tokens, int heads, int dim,
                      float sm_scale, uint16_t* out, void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
