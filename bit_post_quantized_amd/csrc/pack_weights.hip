// Residual weight quantization and nibble packing (offline weight preparation).
//
// Residual quantization of the SVD split (FLUX4 2.2 "three steps", third step) with the
// symmetric b-bit rule of W4A8 3.1 at b = 4, per (64-group of k, output column n).
// One thread owns one (g, n): it reads the 64 values R[g*64 .. g*64+63][n] (coalesced across
// the threads of a row of R), finds the group max, derives the fp16 scale, codes the values
// and writes 32 packed bytes to wq[n][g*32 ..] as two 16-byte stores.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

__global__ __launch_bounds__(256) void pack_weights_kernel(const float* __restrict__ R, int K,
                                                           int N, uint8_t* __restrict__ wq,
                                                           uint16_t* __restrict__ w_scales) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int g = blockIdx.y;
  if (n >= N) return;
  const float* col = R + (size_t)g * kGroup * N + n;
  float v[kGroup];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    v[i] = col[(size_t)i * N];
    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
  const uint16_t sb = int4_scale_bits(amax);
  const float s = half_bits_to_float(sb);
  uint32_t packed[8];
  quantize_group_int4(v, s, packed);
  v4u* dst = reinterpret_cast<v4u*>(wq + (size_t)n * (K / 2) + (size_t)g * (kGroup / 2));
  dst[0] = v4u{packed[0], packed[1], packed[2], packed[3]};
  dst[1] = v4u{packed[4], packed[5], packed[6], packed[7]};
  w_scales[(size_t)g * N + n] = sb;
}

hipError_t launch_pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                               hipStream_t stream) {
  dim3 grid((N + 255) / 256, K / kGroup);
  hipLaunchKernelGGL(pack_weights_kernel, grid, dim3(256), 0, stream, R, K, N, wq, w_scales);
  return hipGetLastError();
}

}  // namespace svdq
