// Residual weight quantization and packing (offline weight preparation).
//
// Residual quantization of the SVD split (FLUX4 2.2 "three steps", third step) with the
// symmetric b-bit rule of W4A8 3.1 at b = 4, per (64-group of k, output column n).
// One thread owns one (g, n): it reads the 64 values R[g*64 .. g*64+63][n] (coalesced across
// the threads of a row of R), finds the group max, derives the fp16 scale, codes the values
// and writes them to row n of wq as 32 bytes of nibbles, or as two 24-byte slots of the tiled
// BF6 (E3M2) container (block n / 32, group g, slots n % 32 and 32 + n % 32).  For the tiled
// container the grid covers columns up to the next multiple of 32 and writes zero codes there.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

template <bool E3M2>
__global__ __launch_bounds__(256) void pack_weights_kernel(const float* __restrict__ R, int K,
                                                           int N, uint8_t* __restrict__ wq,
                                                           uint16_t* __restrict__ w_scales) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int g = blockIdx.y;
  const int n_end = E3M2 ? (N + kE3m2Rows - 1) / kE3m2Rows * kE3m2Rows : N;
  if (n >= n_end) return;
  const bool live = n < N;
  const float* col = R + (size_t)g * kGroup * N + (live ? n : 0);
  float v[kGroup];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    v[i] = live ? col[(size_t)i * N] : 0.0f;
    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
  const uint16_t sb = int4_scale_bits(amax);
  const float s = half_bits_to_float(sb);
  const bool zero = s == 0.0f;
  const float s1 = zero ? 1.0f : s;
  const float rcp = 1.0f / s1;
  float c[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float q = __builtin_amdgcn_fmed3f(rne_quotient(v[i], s1, rcp), -8.0f, 7.0f);
    c[i] = zero ? 0.0f : q + 0.0f;  // + 0 turns a -0 code into +0
  }
  if constexpr (E3M2) {
    uint32_t w[12];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v3u p = pack16_e3m2(c + 16 * j);
      w[3 * j] = p.x;
      w[3 * j + 1] = p.y;
      w[3 * j + 2] = p.z;
    }
    uint8_t* blk = wq + ((size_t)(n >> 5) * (K / kGroup) + g) * kE3m2Block;
    v2u* s0 = reinterpret_cast<v2u*>(blk + (n & 31) * 24);         // codes k = 0..31
    v2u* s1 = reinterpret_cast<v2u*>(blk + (32 + (n & 31)) * 24);  // codes k = 32..63
    s0[0] = v2u{w[0], w[1]};
    s0[1] = v2u{w[2], w[3]};
    s0[2] = v2u{w[4], w[5]};
    s1[0] = v2u{w[6], w[7]};
    s1[1] = v2u{w[8], w[9]};
    s1[2] = v2u{w[10], w[11]};
  } else {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = pack8_nibbles(c + 8 * j);
    v4u* dst = reinterpret_cast<v4u*>(wq + (size_t)n * (K / 2) + (size_t)g * (kGroup / 2));
    dst[0] = v4u{w[0], w[1], w[2], w[3]};
    dst[1] = v4u{w[4], w[5], w[6], w[7]};
  }
  if (live) w_scales[(size_t)g * N + n] = sb;
}

hipError_t launch_pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                               int e3m2, hipStream_t stream) {
  const int cols = e3m2 ? (N + kE3m2Rows - 1) / kE3m2Rows * kE3m2Rows : N;
  dim3 grid((cols + 255) / 256, K / kGroup);
  if (e3m2)
    hipLaunchKernelGGL(pack_weights_kernel<true>, grid, dim3(256), 0, stream, R, K, N, wq, w_scales);
  else
    hipLaunchKernelGGL(pack_weights_kernel<false>, grid, dim3(256), 0, stream, R, K, N, wq, w_scales);
  return hipGetLastError();
}

// Low-rank factor relayouts (offline weight preparation, like the residual packing above), for
// the two factors of the 16-bit branch (SVDQ "technical principles"): L1 [K, r] becomes
// [r, K], each rank's K values contiguous, the layout the activation pass reads (one row's
// 64-value group slice of a rank per 16-byte pair); L2 [r, N] becomes [N, r], each column's
// ranks contiguous, the layout the GEMM epilogue reads (8 ranks of a column per 16-byte
// fragment).  Plain transposes through LDS in 64 x 64 tiles (bf16 values copied, no
// arithmetic).
// bf16 transpose dst [cols, rows] = src [rows, cols]^T through a 64 x 65 LDS tile (both the
// loads and the stores coalesced); block (x, y) covers columns 64 x and rows 64 y
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             int rows, int cols,
                                                             uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;  // coalesced along a row of src
    if (r0 + rr < rows && c0 + cc < cols) tile[rr][cc] = src[(size_t)(r0 + rr) * cols + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;  // coalesced along a row of dst
    if (r0 + rr < rows && c0 + cc < cols) dst[(size_t)(c0 + cc) * rows + r0 + rr] = tile[rr][cc];
  }
}

static hipError_t launch_transpose(const uint16_t* src, int rows, int cols, uint16_t* dst,
                                   hipStream_t stream) {
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, src, rows, cols, dst);
  return hipGetLastError();
}

// L1 [K, r] -> L1p [r, K]
hipError_t launch_pack_lowrank(const uint16_t* L1, int K, int r, uint16_t* L1p,
                               hipStream_t stream) {
  return launch_transpose(L1, K, r, L1p, stream);
}

// L2 [r, N] -> L2p [N, r]
hipError_t launch_pack_lowrank_up(const uint16_t* L2, int r, int N, uint16_t* L2p,
                                  hipStream_t stream) {
  return launch_transpose(L2, r, N, L2p, stream);
}

}  // namespace svdq
