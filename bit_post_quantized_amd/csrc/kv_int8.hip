// Asymmetric per-channel INT8 quantization of a KV-cache tensor and its inverse.
//
// VARC "INT8 KV cache quantization": per-channel INT8 with a non-centered zero point, because
// the cache is skewed and its variance is driven by particular channels.  A channel is one
// (head, dim) pair of x [tokens, channels]; its statistics run over every token of the call,
// so quantization needs a cross-token reduction before the codes can be written:
//   1. kv_range_kernel: each block reduces a chunk of tokens for 2048 channels to a partial
//      (min, max), starting from 0 so the range always contains 0;
//   2. kv_params_kernel: one thread per channel folds the chunk partials and derives
//      s = fl32(fl32(hi - lo) / 255) (1 if 0) and z = clamp(rne(fl32(-lo / s)), 0, 255);
//   3. kv_quant_kernel: re-reads the chunk (the tensor is small enough to still sit in the
//      256 MB last-level cache) and writes q = clamp(rne(fl32(x / s)) + z, 0, 255).
// Thread layout: one thread per 8 consecutive channels (one 16-byte load per token row), so a
// wave reads 1 KB of a row contiguously and the per-channel reduction needs no shuffles.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

constexpr int kKvThreads = 256;        // channel groups (of 8) per block
constexpr int kKvRowsPerChunk = 64;   // tokens per block in the range and quantize passes

__device__ __forceinline__ void decode8_bf16(const v4u w, float* v) {
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xFFFF0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  v[4] = __uint_as_float(w.z << 16);
  v[5] = __uint_as_float(w.z & 0xFFFF0000u);
  v[6] = __uint_as_float(w.w << 16);
  v[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

__global__ __launch_bounds__(kKvThreads) void kv_range_kernel(const uint16_t* __restrict__ x,
                                                              int tokens, int channels,
                                                              float* __restrict__ ws_lo,
                                                              float* __restrict__ ws_hi) {
  const int cg = blockIdx.x * kKvThreads + threadIdx.x;
  if (cg >= channels / 8) return;
  const int chunk = blockIdx.y;
  const int t0 = chunk * kKvRowsPerChunk;
  const int t1 = min(tokens, t0 + kKvRowsPerChunk);
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
  const uint16_t* p = x + (size_t)t0 * channels + (size_t)cg * 8;
#pragma unroll 8
  for (int t = t0; t < t1; ++t, p += channels) {
    float v[8];
    decode8_bf16(*reinterpret_cast<const v4u*>(p), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = __builtin_fminf(lo[i], v[i]);
      hi[i] = __builtin_fmaxf(hi[i], v[i]);
    }
  }
  v4f* dl = reinterpret_cast<v4f*>(ws_lo + (size_t)chunk * channels + (size_t)cg * 8);
  v4f* dh = reinterpret_cast<v4f*>(ws_hi + (size_t)chunk * channels + (size_t)cg * 8);
  dl[0] = v4f{lo[0], lo[1], lo[2], lo[3]};
  dl[1] = v4f{lo[4], lo[5], lo[6], lo[7]};
  dh[0] = v4f{hi[0], hi[1], hi[2], hi[3]};
  dh[1] = v4f{hi[4], hi[5], hi[6], hi[7]};
}

__global__ __launch_bounds__(256) void kv_params_kernel(const float* __restrict__ ws_lo,
                                                        const float* __restrict__ ws_hi,
                                                        int nchunks, int channels,
                                                        float* __restrict__ scale,
                                                        uint8_t* __restrict__ zero) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= channels) return;
  float lo = 0.0f, hi = 0.0f;
  for (int k = 0; k < nchunks; ++k) {
    lo = __builtin_fminf(lo, ws_lo[(size_t)k * channels + c]);
    hi = __builtin_fmaxf(hi, ws_hi[(size_t)k * channels + c]);
  }
  float s = (hi - lo) / 255.0f;
  if (s == 0.0f) s = 1.0f;
  const float z = rne_quotient(-lo, s, 1.0f / s);
  scale[c] = s;
  zero[c] = (uint8_t)__builtin_fminf(__builtin_fmaxf(z, 0.0f), 255.0f);
}

__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(const uint16_t* __restrict__ x,
                                                              int tokens, int channels,
                                                              const float* __restrict__ scale,
                                                              const uint8_t* __restrict__ zero,
                                                              uint8_t* __restrict__ q) {
  const int cg = blockIdx.x * kKvThreads + threadIdx.x;
  if (cg >= channels / 8) return;
  const int t0 = blockIdx.y * kKvRowsPerChunk;
  const int t1 = min(tokens, t0 + kKvRowsPerChunk);
  float s[8], rcp[8], z[8];
  {
    const v4f s0 = reinterpret_cast<const v4f*>(scale + (size_t)cg * 8)[0];
    const v4f s1 = reinterpret_cast<const v4f*>(scale + (size_t)cg * 8)[1];
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    const v2u zz = *reinterpret_cast<const v2u*>(zero + (size_t)cg * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rcp[i] = 1.0f / s[i];
      z[i] = (float)(((i < 4 ? zz.x : zz.y) >> (8 * (i & 3))) & 0xFFu);
    }
  }
  const uint16_t* p = x + (size_t)t0 * channels + (size_t)cg * 8;
  uint8_t* d = q + (size_t)t0 * channels + (size_t)cg * 8;
#pragma unroll 4
  for (int t = t0; t < t1; ++t, p += channels, d += channels) {
    float v[8];
    decode8_bf16(*reinterpret_cast<const v4u*>(p), v);
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = rne_quotient(v[i], s[i], rcp[i]) + z[i];
      c = __builtin_fminf(__builtin_fmaxf(c, 0.0f), 255.0f);
      if (i < 4)
        w0 |= (uint32_t)c << (8 * i);
      else
        w1 |= (uint32_t)c << (8 * (i - 4));
    }
    *reinterpret_cast<v2u*>(d) = v2u{w0, w1};
  }
}

__global__ __launch_bounds__(kKvThreads) void kv_dequant_kernel(const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scale,
                                                                const uint8_t* __restrict__ zero,
                                                                int tokens, int channels,
                                                                uint16_t* __restrict__ out) {
  const int cg = blockIdx.x * kKvThreads + threadIdx.x;
  if (cg >= channels / 8) return;
  const int t0 = blockIdx.y * kKvRowsPerChunk;
  const int t1 = min(tokens, t0 + kKvRowsPerChunk);
  float s[8], z[8];
  {
    const v4f s0 = reinterpret_cast<const v4f*>(scale + (size_t)cg * 8)[0];
    const v4f s1 = reinterpret_cast<const v4f*>(scale + (size_t)cg * 8)[1];
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    const v2u zz = *reinterpret_cast<const v2u*>(zero + (size_t)cg * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (float)(((i < 4 ? zz.x : zz.y) >> (8 * (i & 3))) & 0xFFu);
  }
  const uint8_t* p = q + (size_t)t0 * channels + (size_t)cg * 8;
  uint16_t* d = out + (size_t)t0 * channels + (size_t)cg * 8;
#pragma unroll 4
  for (int t = t0; t < t1; ++t, p += channels, d += channels) {
    const v2u w = *reinterpret_cast<const v2u*>(p);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = (float)(((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu);
      v[i] = (c - z[i]) * s[i];  // (q - z) is an exact small integer in fp32
    }
    *reinterpret_cast<v4u*>(d) = v4u{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                     pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7])};
  }
}

static inline int kv_chunks(int tokens) { return (tokens + kKvRowsPerChunk - 1) / kKvRowsPerChunk; }

size_t kv_workspace_bytes(int tokens, int channels) {
  if (tokens <= 0 || channels <= 0) return 0;
  return (size_t)2 * kv_chunks(tokens) * channels * sizeof(float);
}

hipError_t launch_kv_quant(const uint16_t* x, int tokens, int channels, uint8_t* q,
                           float* scale, uint8_t* zero, void* workspace, hipStream_t stream) {
  const int nchunks = kv_chunks(tokens);
  float* ws_lo = reinterpret_cast<float*>(workspace);
  float* ws_hi = ws_lo + (size_t)nchunks * channels;
  const dim3 grid((channels / 8 + kKvThreads - 1) / kKvThreads, nchunks);
  hipLaunchKernelGGL(kv_range_kernel, grid, dim3(kKvThreads), 0, stream, x, tokens, channels,
                     ws_lo, ws_hi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_params_kernel, dim3((channels + 255) / 256), dim3(256), 0, stream, ws_lo,
                     ws_hi, nchunks, channels, scale, zero);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_quant_kernel, grid, dim3(kKvThreads), 0, stream, x, tokens, channels,
                     scale, zero, q);
  return hipGetLastError();
}

hipError_t launch_kv_dequant(const uint8_t* q, const float* scale, const uint8_t* zero,
                             int tokens, int channels, uint16_t* x_out, hipStream_t stream) {
  const dim3 grid((channels / 8 + kKvThreads - 1) / kKvThreads, kv_chunks(tokens));
  hipLaunchKernelGGL(kv_dequant_kernel, grid, dim3(kKvThreads), 0, stream, q, scale, zero,
                     tokens, channels, x_out);
  return hipGetLastError();
}

}  // namespace svdq
