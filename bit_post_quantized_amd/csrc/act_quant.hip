// Fused activation pass: smoothing, dynamic INT4 quantization and the low-rank down-projection.
//
// SVDQ "technical principles": smoothing moves activation outliers into the weights, and a
// 16-bit low-rank branch runs beside the 4-bit one.  FLUX4 3.1: activations are quantized at
// run time.  W4A8 3.1: symmetric scale max|v| / (2^(b-1) - 1), round, clamp (b = 4 here, one
// scale per token and 64-group).  SVDQ / DCMP: the branch is fused so the activations are read
// from HBM once.
//
// Work decomposition.  A workgroup owns 16 tokens (rows).  K is cut into strips of 256
// (four 64-groups); the (up to 8) waves of the workgroup take strips round-robin.  Inside a strip, lane
// l holds row (l % 16) and group (l / 16) of the strip: it loads that group's 64 bf16 values
// (128 contiguous bytes), smooths them, finds the group max in-lane (no shuffles), quantizes and
// writes its 32 packed bytes and its scale.  The same registers, rounded to bf16, are the A
// operand of v_mfma_f32_16x16x32_bf16: in MFMA step j (0..7) lane group q supplies k = 64q+8j+i,
// and the B operand (L1, stored K-contiguous) is loaded with the same k map, so the 8 MFMAs of
// a strip sum exactly the strip's 256 k.  Per-wave partial T tiles are summed in LDS in wave
// order (deterministic) and written once.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

template <int NTR>  // number of 16-wide tiles of the rank r (r = 16 * NTR)
__global__ __launch_bounds__(512) void quantize_act_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ inv_lambda,
    const uint16_t* __restrict__ L1, int M, int K, uint8_t* __restrict__ xq,
    uint16_t* __restrict__ x_scales, float* __restrict__ T) {
  extern __shared__ float red[];  // [nwaves][16][r]
  constexpr int r = 16 * NTR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int rl = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + rl;
  const int row_ld = row < M ? row : M - 1;
  const int G = K / kGroup;
  const int nstrips = (G + 3) / 4;

  v4f acc[NTR > 0 ? NTR : 1];
#pragma unroll
  for (int t = 0; t < (NTR > 0 ? NTR : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int strip = wave; strip < nstrips; strip += nwaves) {
    const int g = strip * 4 + q;
    const bool valid = g < G;
    const int k0 = (valid ? g : G - 1) * kGroup;  // loads stay in bounds; invalid lanes zeroed
    float xh[kGroup];
    {
      const v4u* xs = reinterpret_cast<const v4u*>(X + (size_t)row_ld * K + k0);
      const v4f* ls = reinterpret_cast<const v4f*>(inv_lambda + k0);
      const float keep = valid ? 1.0f : 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v4u w = xs[c];
        const v4f l0 = ls[2 * c] * keep, l1 = ls[2 * c + 1] * keep;
        xh[8 * c + 0] = __uint_as_float(w.x << 16) * l0.x;
        xh[8 * c + 1] = __uint_as_float(w.x & 0xFFFF0000u) * l0.y;
        xh[8 * c + 2] = __uint_as_float(w.y << 16) * l0.z;
        xh[8 * c + 3] = __uint_as_float(w.y & 0xFFFF0000u) * l0.w;
        xh[8 * c + 4] = __uint_as_float(w.z << 16) * l1.x;
        xh[8 * c + 5] = __uint_as_float(w.z & 0xFFFF0000u) * l1.y;
        xh[8 * c + 6] = __uint_as_float(w.w << 16) * l1.z;
        xh[8 * c + 7] = __uint_as_float(w.w & 0xFFFF0000u) * l1.w;
      }
    }

    // ---- INT4 quantization of this lane's group
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[i]));
    const uint16_t sb = int4_scale_bits(amax);
    const float s = half_bits_to_float(sb);
    uint32_t packed[8];
    quantize_group_int4(xh, s, packed);
    if (valid && row < M) {
      v4u* dst = reinterpret_cast<v4u*>(xq + (size_t)row * (K / 2) + (size_t)g * (kGroup / 2));
      dst[0] = v4u{packed[0], packed[1], packed[2], packed[3]};
      dst[1] = v4u{packed[4], packed[5], packed[6], packed[7]};
      x_scales[(size_t)g * M + row] = sb;
    }

    // ---- low-rank down-projection on bf16 MFMA
    if constexpr (NTR > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v4u a;
        a.x = pack2_bf16(xh[8 * j + 0], xh[8 * j + 1]);
        a.y = pack2_bf16(xh[8 * j + 2], xh[8 * j + 3]);
        a.z = pack2_bf16(xh[8 * j + 4], xh[8 * j + 5]);
        a.w = pack2_bf16(xh[8 * j + 6], xh[8 * j + 7]);
        const v8bf av = __builtin_bit_cast(v8bf, a);
#pragma unroll
        for (int t = 0; t < NTR; ++t) {
          const v4u b = *reinterpret_cast<const v4u*>(L1 + (size_t)(t * 16 + rl) * K + k0 + 8 * j);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, b), acc[t], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (NTR > 0) {
    // D layout of a 16x16 MFMA tile: lane l holds column l % 16 and rows 4 * (l / 16) + i.
#pragma unroll
    for (int t = 0; t < NTR; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[((size_t)wave * 16 + 4 * q + i) * r + t * 16 + rl] = acc[t][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * r; idx += blockDim.x) {
      const int rr = idx / r;
      float sum = 0.0f;
      for (int w = 0; w < nwaves; ++w) sum += red[(size_t)w * 16 * r + idx];
      if (row0 + rr < M) T[(size_t)(row0 + rr) * r + (idx % r)] = sum;
    }
  }
}

hipError_t launch_quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                               int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                               hipStream_t stream) {
  const int G = K / kGroup;
  const int nstrips = (G + 3) / 4;
  // up to 8 waves; prefer a count that divides the strips evenly (12 strips -> 6 waves)
  int nwaves = nstrips < 8 ? nstrips : 8;
  for (int d = nwaves; d >= 4; --d)
    if (nstrips % d == 0) {
      nwaves = d;
      break;
    }
  const size_t lds = (size_t)nwaves * 16 * r * sizeof(float);
  dim3 grid((M + 15) / 16), block(64 * nwaves);
  switch (r / 16) {
#define SVDQ_ACT_CASE(n)                                                                  \
  case n:                                                                                 \
    hipLaunchKernelGGL(quantize_act_kernel<n>, grid, block, lds, stream, X, inv_lambda, L1, \
                       M, K, xq, x_scales, T);                                            \
    break;
    SVDQ_ACT_CASE(0)
    SVDQ_ACT_CASE(1)
    SVDQ_ACT_CASE(2)
    SVDQ_ACT_CASE(3)
    SVDQ_ACT_CASE(4)
    SVDQ_ACT_CASE(5)
    SVDQ_ACT_CASE(6)
    SVDQ_ACT_CASE(7)
    SVDQ_ACT_CASE(8)
#undef SVDQ_ACT_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svdq
