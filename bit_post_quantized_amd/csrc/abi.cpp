// C ABI of libsvdq (declared in include/svdq.h): argument validation and kernel dispatch.
//
// Every entry point checks all of its arguments before touching the HIP runtime, so a
// rejected call has no side effect at all (no launch, no device state, outputs untouched).
#include "svdq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "svdq_launch.hpp"

namespace {

thread_local char g_last_error[256] = {0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = 0;
  return SVDQ_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SVDQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr long long kMaxElems = 1LL << 40;  // keeps every byte offset far inside size_t
constexpr int kMaxRank = 128;
// The KV dequantization's grid holds the tokens in its y dimension, at most 65535 blocks of 32.
constexpr int kKvMaxTokens = 65535 * 32;

int check_k(int K) {
  if (K <= 0) return fail(SVDQ_EINVAL, "K must be positive (got %d)", K);
  if (K % 64 != 0) return fail(SVDQ_ESHAPE, "K must be a multiple of 64 (got %d)", K);
  return SVDQ_OK;
}

int check_rank(int r) {
  if (r < 0) return fail(SVDQ_EINVAL, "r must be >= 0 (got %d)", r);
  if (r % 16 != 0 || r > kMaxRank)
    return fail(SVDQ_ESHAPE, "r must be a multiple of 16 in [0, %d] (got %d)", kMaxRank, r);
  return SVDQ_OK;
}

}  // namespace

extern "C" {

int svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

const char* svdq_status_str(int status) {
  switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_EINVAL: return "invalid argument";
    case SVDQ_ESHAPE: return "unsupported shape";
    case SVDQ_EALIGN: return "misaligned pointer";
    case SVDQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* svdq_last_error(void) { return g_last_error; }

static int pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                        void* stream, int e3m2, const char* name) {
  if (int s = check_k(K)) return s;
  if (N <= 0) return fail(SVDQ_EINVAL, "N must be positive (got %d)", N);
  if ((long long)K * N > kMaxElems) return fail(SVDQ_ESHAPE, "K * N too large");
  if (K / 64 > 65535) return fail(SVDQ_ESHAPE, "K / 64 must be <= 65535");
  if (!R || !wq || !w_scales) return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(R) || !aligned16(wq)) return fail(SVDQ_EALIGN, "R and wq must be 16-byte aligned");
  return hip_status(svdq::launch_pack_weights(R, K, N, wq, w_scales, e3m2, (hipStream_t)stream),
                    name);
}

int svdq_pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                      void* stream) {
  return pack_weights(R, K, N, wq, w_scales, stream, 0, "svdq_pack_weights");
}

int svdq_pack_weights_e3m2(const float* R, int K, int N, uint8_t* wq6, uint16_t* w_scales,
                           void* stream) {
  return pack_weights(R, K, N, wq6, w_scales, stream, 1, "svdq_pack_weights_e3m2");
}

int svdq_pack_lowrank(const uint16_t* L1, int K, int r, uint16_t* L1p, void* stream) {
  if (int s = check_k(K)) return s;
  if (int s = check_rank(r)) return s;
  if (r == 0) return fail(SVDQ_ESHAPE, "r must be positive for the factor relayout");
  if (K / 64 > 65535) return fail(SVDQ_ESHAPE, "K / 64 must be <= 65535");
  if (!L1 || !L1p) return fail(SVDQ_EINVAL, "NULL pointer");
  return hip_status(svdq::launch_pack_lowrank(L1, K, r, L1p, (hipStream_t)stream),
                    "svdq_pack_lowrank");
}

int svdq_pack_lowrank_up(const uint16_t* L2, int r, int N, uint16_t* L2p, void* stream) {
  if (int s = check_rank(r)) return s;
  if (r == 0) return fail(SVDQ_ESHAPE, "r must be positive for the factor relayout");
  if (N <= 0) return fail(SVDQ_EINVAL, "N must be positive (got %d)", N);
  if (N > (1 << 24)) return fail(SVDQ_ESHAPE, "N must be <= 2^24 (got %d)", N);
  if (!L2 || !L2p) return fail(SVDQ_EINVAL, "NULL pointer");
  return hip_status(svdq::launch_pack_lowrank_up(L2, r, N, L2p, (hipStream_t)stream),
                    "svdq_pack_lowrank_up");
}

static int quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1, int M,
                        int K, int r, uint8_t* xq, uint16_t* x_scales, float* T, void* stream,
                        int codes, const char* name) {
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0 (got %d)", M);
  if (int s = check_k(K)) return s;
  if (int s = check_rank(r)) return s;
  if ((long long)M * K > kMaxElems) return fail(SVDQ_ESHAPE, "M * K too large");
  if (!X || !inv_lambda || !xq || !x_scales) return fail(SVDQ_EINVAL, "NULL pointer");
  if (r > 0 && (!L1 || !T)) return fail(SVDQ_EINVAL, "L1 and T are required when r > 0");
  if (!aligned16(X) || !aligned16(inv_lambda) || !aligned16(xq) || (r > 0 && !aligned16(L1)))
    return fail(SVDQ_EALIGN, "X, inv_lambda, xq and L1 must be 16-byte aligned");
  if (M == 0) return ok();
  return hip_status(svdq::launch_quantize_act(X, inv_lambda, L1, M, K, r, xq, x_scales, T, codes,
                                              (hipStream_t)stream),
                    name);
}

int svdq_quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1, int M,
                      int K, int r, uint8_t* xq, uint16_t* x_scales, float* T, void* stream) {
  return quantize_act(X, inv_lambda, L1, M, K, r, xq, x_scales, T, stream, svdq::kCodesNibbles,
                      "svdq_quantize_act");
}

int svdq_quantize_act_e3m2(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                           int M, int K, int r, uint8_t* xq6, uint16_t* x_scales, float* T,
                           void* stream) {
  return quantize_act(X, inv_lambda, L1, M, K, r, xq6, x_scales, T, stream, svdq::kCodesBf6,
                      "svdq_quantize_act_e3m2");
}

int svdq_quantize_act_a8(const uint16_t* X, const float* inv_lambda, const uint16_t* L1, int M,
                         int K, int r, int8_t* xq8, uint16_t* x_scales, float* T, void* stream) {
  return quantize_act(X, inv_lambda, L1, M, K, r, reinterpret_cast<uint8_t*>(xq8), x_scales, T,
                      stream, svdq::kCodesInt8, "svdq_quantize_act_a8");
}

static int check_gemm(const uint8_t* xq, const uint8_t* wq, int M, int N, int K) {
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0 (got %d)", M);
  if (N <= 0) return fail(SVDQ_EINVAL, "N must be positive (got %d)", N);
  if (int s = check_k(K)) return s;
  if ((long long)M * N > kMaxElems || (long long)M * K > kMaxElems || (long long)N * K > kMaxElems)
    return fail(SVDQ_ESHAPE, "problem too large");
  if (M > 65535 * 128) return fail(SVDQ_ESHAPE, "M too large for one launch");
  // row offsets inside an output tile (< 256 N) are 32-bit in the kernels
  if (N > (1 << 24)) return fail(SVDQ_ESHAPE, "N must be <= 2^24 (got %d)", N);
  if (K / 64 > 65535) return fail(SVDQ_ESHAPE, "K / 64 must be <= 65535 (got K = %d)", K);
  if (!xq || !wq) return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(xq) || !aligned16(wq)) return fail(SVDQ_EALIGN, "xq and wq must be 16-byte aligned");
  return SVDQ_OK;
}

typedef hipError_t (*gemm_launcher)(const uint8_t*, const uint16_t*, const float*,
                                    const uint8_t*, const uint16_t*, const uint16_t*,
                                    const uint16_t*, int, int, int, int, void*, int, int32_t*,
                                    hipStream_t);

static int gemm(gemm_launcher launch, const char* name, const uint8_t* xq,
                const uint16_t* x_scales, const float* T, const uint8_t* wq,
                const uint16_t* w_scales, const uint16_t* L2, const uint16_t* bias, int M, int N,
                int K, int r, void* Y, int out_dtype, void* stream) {
  if (int s = check_gemm(xq, wq, M, N, K)) return s;
  if (int s = check_rank(r)) return s;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_FP32)
    return fail(SVDQ_EINVAL, "out_dtype must be SVDQ_OUT_BF16 or SVDQ_OUT_FP32");
  if (!x_scales || !w_scales || !Y) return fail(SVDQ_EINVAL, "NULL pointer");
  if (r > 0 && (!T || !L2)) return fail(SVDQ_EINVAL, "T and L2 are required when r > 0");
  if (!aligned16(Y) || (r > 0 && (!aligned16(T) || !aligned16(L2))))
    return fail(SVDQ_EALIGN, "Y, T and L2 must be 16-byte aligned");
  if (M == 0) return ok();
  return hip_status(launch(xq, x_scales, T, wq, w_scales, L2, bias, M, N, K, r, Y,
                           out_dtype == SVDQ_OUT_FP32, nullptr, (hipStream_t)stream),
                    name);
}

static int partials(gemm_launcher launch, const char* name, const uint8_t* xq,
                    const uint8_t* wq, int M, int N, int K, int32_t* P, void* stream) {
  if (int s = check_gemm(xq, wq, M, N, K)) return s;
  if (!P) return fail(SVDQ_EINVAL, "NULL pointer");
  if (M == 0) return ok();
  return hip_status(launch(xq, nullptr, nullptr, wq, nullptr, nullptr, nullptr, M, N, K, 0,
                           nullptr, 0, P, (hipStream_t)stream),
                    name);
}

int svdq_w4a4_gemm(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                   const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                   const uint16_t* bias, int M, int N, int K, int r, void* Y, int out_dtype,
                   void* stream) {
  return gemm(svdq::launch_w4a4_gemm, "svdq_w4a4_gemm", xq, x_scales, T, wq, w_scales, L2,
              bias, M, N, K, r, Y, out_dtype, stream);
}

size_t svdq_e3m2_bytes(int rows, int K) {
  if (rows <= 0 || K <= 0 || K % 64 != 0) return 0;
  return (((size_t)rows + 31) / 32) * (size_t)(K / 64) * (64 * 24);
}

int svdq_w4a4_gemm_e3m2(const uint8_t* xq6, const uint16_t* x_scales, const float* T,
                        const uint8_t* wq6, const uint16_t* w_scales, const uint16_t* L2,
                        const uint16_t* bias, int M, int N, int K, int r, void* Y,
                        int out_dtype, void* stream) {
  return gemm(svdq::launch_w4a4_gemm_e3m2, "svdq_w4a4_gemm_e3m2", xq6, x_scales, T, wq6,
              w_scales, L2, bias, M, N, K, r, Y, out_dtype, stream);
}

int svdq_w4a4_partials(const uint8_t* xq, const uint8_t* wq, int M, int N, int K, int32_t* P,
                       void* stream) {
  return partials(svdq::launch_w4a4_gemm, "svdq_w4a4_partials", xq, wq, M, N, K, P, stream);
}

int svdq_w4a4_partials_e3m2(const uint8_t* xq6, const uint8_t* wq6, int M, int N, int K,
                            int32_t* P, void* stream) {
  return partials(svdq::launch_w4a4_gemm_e3m2, "svdq_w4a4_partials_e3m2", xq6, wq6, M, N, K, P,
                  stream);
}

int svdq_w4a8_gemm(const int8_t* xq8, const uint16_t* x_scales, const float* T,
                   const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                   const uint16_t* bias, int M, int N, int K, int r, void* Y, int out_dtype,
                   void* stream) {
  return gemm(svdq::launch_w4a8_gemm, "svdq_w4a8_gemm", reinterpret_cast<const uint8_t*>(xq8),
              x_scales, T, wq, w_scales, L2, bias, M, N, K, r, Y, out_dtype, stream);
}

int svdq_w4a8_partials(const int8_t* xq8, const uint8_t* wq, int M, int N, int K, int32_t* P,
                       void* stream) {
  return partials(svdq::launch_w4a8_gemm, "svdq_w4a8_partials",
                  reinterpret_cast<const uint8_t*>(xq8), wq, M, N, K, P, stream);
}

size_t kv_int8_workspace_bytes(int tokens, int channels) {
  return svdq::kv_workspace_bytes(tokens, channels);
}

static int check_kv(int tokens, int channels) {
  if (tokens < 0) return fail(SVDQ_EINVAL, "tokens must be >= 0 (got %d)", tokens);
  if (channels <= 0) return fail(SVDQ_EINVAL, "channels must be positive (got %d)", channels);
  if (channels % 8 != 0) return fail(SVDQ_ESHAPE, "channels must be a multiple of 8 (got %d)", channels);
  if ((long long)tokens * channels > kMaxElems) return fail(SVDQ_ESHAPE, "tensor too large");
  if (tokens > kKvMaxTokens)
    return fail(SVDQ_ESHAPE, "tokens must be <= %d (got %d)", kKvMaxTokens, tokens);
  return SVDQ_OK;
}

int kv_int8_quant(const uint16_t* x, int tokens, int channels, uint8_t* q, float* scale,
                  uint8_t* zero, void* workspace, void* stream) {
  if (int s = check_kv(tokens, channels)) return s;
  if (!x || !q || !scale || !zero || (tokens > 0 && !workspace))
    return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale) || !aligned16(zero) ||
      !aligned16(workspace))
    return fail(SVDQ_EALIGN, "x, q, scale, zero and workspace must be 16-byte aligned");
  if (tokens == 0) return ok();
  return hip_status(svdq::launch_kv_quant(x, tokens, channels, q, scale, zero, workspace,
                                          (hipStream_t)stream),
                    "kv_int8_quant");
}

int kv_int8_quant_pair(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                       uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv, uint8_t* zv,
                       void* workspace, void* stream) {
  if (int s = check_kv(tokens, channels)) return s;
  if (!k || !v || !qk || !sk || !zk || !qv || !sv || !zv || (tokens > 0 && !workspace))
    return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(qk) || !aligned16(sk) || !aligned16(zk) ||
      !aligned16(qv) || !aligned16(sv) || !aligned16(zv) || !aligned16(workspace))
    return fail(SVDQ_EALIGN, "tensors and workspace must be 16-byte aligned");
  if (tokens == 0) return ok();
  return hip_status(svdq::launch_kv_quant_pair(k, v, tokens, channels, qk, sk, zk, qv, sv, zv,
                                               workspace, (hipStream_t)stream),
                    "kv_int8_quant_pair");
}

int kv_int8_quant_pair_noalloc(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                               uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv,
                               uint8_t* zv, void* stream) {
  if (int s = check_kv(tokens, channels)) return s;
  if (!k || !v || !qk || !sk || !zk || !qv || !sv || !zv) return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(qk) || !aligned16(sk) || !aligned16(zk) ||
      !aligned16(qv) || !aligned16(sv) || !aligned16(zv))
    return fail(SVDQ_EALIGN, "tensors must be 16-byte aligned");
  const size_t need = svdq::kv_workspace_bytes(tokens, channels);
  if (need > svdq::kKvStaticScratchBytes)
    return fail(SVDQ_ESHAPE,
                "tokens %d x channels %d need %zu bytes of scratch; this entry point holds %zu "
                "(use kv_int8_quant_pair with a workspace)",
                tokens, channels, need, svdq::kKvStaticScratchBytes);
  if (tokens == 0) return ok();
  return hip_status(svdq::launch_kv_quant_pair_noalloc(k, v, tokens, channels, qk, sk, zk, qv, sv,
                                                       zv, (hipStream_t)stream),
                    "kv_int8_quant_pair_noalloc");
}

int kv_int8_dequant(const uint8_t* q, const float* scale, const uint8_t* zero, int tokens,
                    int channels, uint16_t* x_out, void* stream) {
  if (int s = check_kv(tokens, channels)) return s;
  if (!q || !scale || !zero || !x_out) return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(scale) || !aligned16(zero) || !aligned16(x_out))
    return fail(SVDQ_EALIGN, "q, scale, zero and x_out must be 16-byte aligned");
  if (tokens == 0) return ok();
  return hip_status(svdq::launch_kv_dequant(q, scale, zero, tokens, channels, x_out,
                                            (hipStream_t)stream),
                    "kv_int8_dequant");
}

size_t kv_int8_attention_workspace_bytes(int nq, int tokens, int heads, int dim) {
  return svdq::kv_attn_workspace_bytes(nq, tokens, heads, dim);
}

int kv_int8_attention(const uint16_t* q, const uint8_t* k_codes, const float* k_scale,
                      const uint8_t* k_zero, const uint8_t* v_codes, const float* v_scale,
                      const uint8_t* v_zero, int nq, int tokens, int heads, int dim,
                      float sm_scale, uint16_t* out, void* workspace, void* stream) {
  if (nq <= 0 || tokens <= 0 || heads <= 0)
    return fail(SVDQ_EINVAL, "nq, tokens and heads must be positive (got %d, %d, %d)", nq, tokens,
                heads);
  if (dim != 64 && dim != 128) return fail(SVDQ_ESHAPE, "dim must be 64 or 128 (got %d)", dim);
  // (each bound is checked before a product that could overflow uses it)
  if (nq > 65535 || heads > 65535 || tokens > 4096 * 256 ||
      (long long)tokens * heads * dim > kMaxElems)
    return fail(SVDQ_ESHAPE, "problem too large (at most 1048576 tokens)");
  if (!q || !k_codes || !k_scale || !k_zero || !v_codes || !v_scale || !v_zero || !out ||
      !workspace)
    return fail(SVDQ_EINVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scale) ||
      !aligned16(k_zero) || !aligned16(workspace))
    return fail(SVDQ_EALIGN, "q, codes, k_scale, k_zero and workspace must be 16-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f)
    return fail(SVDQ_EINVAL, "sm_scale must be finite");
  return hip_status(svdq::launch_kv_attention(q, k_codes, k_scale, k_zero, v_codes, v_scale,
                                              v_zero, nq, tokens, heads, dim, sm_scale, out,
                                              workspace, (hipStream_t)stream),
                    "kv_int8_attention");
}

}  // extern "C"
