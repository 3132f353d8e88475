// W4A4 group GEMM with the low-rank up-projection and bias fused into the epilogue.
//
// SVDQ "technical principles" / DCMP "SVDQuant": the 16-bit low-rank branch is fused into the
// low-bit kernel so it costs no extra pass over the activations.  W4A8 2.2 / 4.2: 4-bit
// weights are widened to 8 bits and fed to the INT8 units.  Per 64-group g of K the int32
// partial P[g] = qx[:, g] . qw[g, :] is exact, and
//     Y = sum_g diag(s_x[g]) P[g] diag(s_w[g]) + bf16(T) L2 + bias.
//
// gfx950 mapping.  A 256-thread workgroup computes a 128x128 tile of Y; each of its 4 waves a
// 64x64 sub-tile made of 4x4 tiles of v_mfma_i32_16x16x64_i8.  One MFMA covers exactly one
// group (K = 64), so each MFMA result is one P[g] tile: it is converted, scaled by
// s_x[m] * s_w[n] and accumulated in fp32 registers.  Operands come straight from global memory:
// lane l reads the 8 packed bytes (16 codes) of row/column l % 16 at k-chunk l / 16 and unpacks
// them with the x16 trick (see unpack16_x16), so the MFMA yields 256 * P; the 2^-8 is folded
// into the weight scale (exact).  After the last group, bf16(T) [16 x 32] and L2 [32 x 16]
// fragments go through v_mfma_f32_16x16x32_bf16 with the fp32 accumulator as C, then the bias
// is added and the tile is rounded to bf16 (or kept fp32) and stored.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

constexpr int BM = 128, BN = 128;

template <bool OUT_FP32, bool PARTIALS, int NTR>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ x_scales,
    const float* __restrict__ T, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ w_scales, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, int M, int N, int K, void* __restrict__ Y,
    int32_t* __restrict__ P) {
  constexpr int r = 16 * NTR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = lane & 15;
  const int kc = lane >> 4;
  const int m0 = blockIdx.y * BM + (wave >> 1) * 64;
  const int n0 = blockIdx.x * BN + (wave & 1) * 64;
  const int G = K / kGroup;
  const size_t ldq = (size_t)(K / 2);

  // operand rows / columns owned by this lane (clamped so every load stays in bounds)
  const uint8_t* arow[4];
  const uint8_t* bcol[4];
  int srow[4][4];  // output rows of this lane: m0 + 16 i + 4 kc + e
  int scol[4];     // output columns of this lane: n0 + 16 j + rl
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = min(m0 + 16 * i + rl, M - 1);
    arow[i] = xq + (size_t)ra * ldq + kc * 8;
    const int cb = min(n0 + 16 * i + rl, N - 1);
    bcol[i] = wq + (size_t)cb * ldq + kc * 8;
    scol[i] = n0 + 16 * i + rl;
#pragma unroll
    for (int e = 0; e < 4; ++e) srow[i][e] = m0 + 16 * i + 4 * kc + e;
  }

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < G; ++g) {
    v4i A[4], B[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[i] = unpack16_x16(*reinterpret_cast<const v2u*>(arow[i] + g * 32));
      B[i] = unpack16_x16(*reinterpret_cast<const v2u*>(bcol[i] + g * 32));
    }
    if constexpr (PARTIALS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], B[j], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (srow[i][e] < M && scol[j] < N)
              P[((size_t)g * M + srow[i][e]) * N + scol[j]] = p[e] >> 8;  // exact: 256 * P
        }
    } else {
      float sx[4][4], sw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sx[i][e] = half_bits_to_float(x_scales[(size_t)g * M + min(srow[i][e], M - 1)]);
        sw[i] = half_bits_to_float(w_scales[(size_t)g * N + min(scol[i], N - 1)]) * 0x1p-8f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], B[j], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][e] = __builtin_fmaf((float)p[e], sx[i][e] * sw[j], acc[i][j][e]);
        }
    }
  }
  if constexpr (PARTIALS) return;

  // ---- fused epilogue: low-rank up-projection (bf16 MFMA, fp32 accumulator as C) and bias
  if constexpr (NTR > 0) {
#pragma unroll
    for (int rk = 0; rk < (r + 31) / 32; ++rk) {
      const int kk = rk * 32 + kc * 8;  // this lane's 8 rank indices
      const bool kv = kk < r;
      v8bf At[4], Bt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4u a = v4u{0u, 0u, 0u, 0u}, b = v4u{0u, 0u, 0u, 0u};
        if (kv) {
          const v4f* tp = reinterpret_cast<const v4f*>(T + (size_t)min(m0 + 16 * i + rl, M - 1) * r + kk);
          const v4f t0 = tp[0], t1 = tp[1];
          a = v4u{pack2_bf16(t0.x, t0.y), pack2_bf16(t0.z, t0.w), pack2_bf16(t1.x, t1.y),
                  pack2_bf16(t1.z, t1.w)};
          b = *reinterpret_cast<const v4u*>(L2 + (size_t)min(n0 + 16 * i + rl, N - 1) * r + kk);
        }
        At[i] = __builtin_bit_cast(v8bf, a);
        Bt[i] = __builtin_bit_cast(v8bf, b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(At[i], Bt[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float bj = bias ? bf16_bits_to_float(bias[min(scol[j], N - 1)]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = srow[i][e], col = scol[j];
        if (row < M && col < N) {
          const float v = acc[i][j][e] + bj;
          if constexpr (OUT_FP32)
            reinterpret_cast<float*>(Y)[(size_t)row * N + col] = v;
          else
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * N + col] = float_to_bf16_bits(v);
        }
      }
  }
}

template <bool OUT_FP32, bool PARTIALS>
static hipError_t launch_ntr(int ntr, dim3 grid, hipStream_t stream, const uint8_t* xq,
                             const uint16_t* x_scales, const float* T, const uint8_t* wq,
                             const uint16_t* w_scales, const uint16_t* L2, const uint16_t* bias,
                             int M, int N, int K, void* Y, int32_t* P) {
  switch (ntr) {
#define SVDQ_GEMM_CASE(n)                                                                    \
  case n:                                                                                    \
    hipLaunchKernelGGL((w4a4_gemm_kernel<OUT_FP32, PARTIALS, n>), grid, dim3(256), 0, stream, \
                       xq, x_scales, T, wq, w_scales, L2, bias, M, N, K, Y, P);              \
    break;
    SVDQ_GEMM_CASE(0)
    SVDQ_GEMM_CASE(1)
    SVDQ_GEMM_CASE(2)
    SVDQ_GEMM_CASE(3)
    SVDQ_GEMM_CASE(4)
    SVDQ_GEMM_CASE(5)
    SVDQ_GEMM_CASE(6)
    SVDQ_GEMM_CASE(7)
    SVDQ_GEMM_CASE(8)
#undef SVDQ_GEMM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                            const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                            const uint16_t* bias, int M, int N, int K, int r, void* Y,
                            int out_fp32, int32_t* partials, hipStream_t stream) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (partials)
    return launch_ntr<false, true>(0, grid, stream, xq, nullptr, nullptr, wq, nullptr, nullptr,
                                   nullptr, M, N, K, nullptr, partials);
  if (out_fp32)
    return launch_ntr<true, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2, bias,
                                   M, N, K, Y, nullptr);
  return launch_ntr<false, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2, bias,
                                  M, N, K, Y, nullptr);
}

}  // namespace svdq
