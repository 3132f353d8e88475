// Asymmetric per-channel INT8 quantization of a KV-cache tensor and its inverse.
//
// VARC "INT8 KV cache quantization": per-channel INT8 with a non-centered zero point, because
// the cache is skewed and its variance is driven by particular channels.  A channel is one
// (head, dim) pair of x [tokens, channels]; its statistics run over every token of the call,
// so no code can be written before a cross-token reduction has finished:
//     lo = min(0, min_t x),  hi = max(0, max_t x),
//     s = fl32(fl32(hi - lo) / 255) (1 if 0),  z = clamp(rne(fl32(-lo / s)), 0, 255),
//     q = clamp(rne(fl32(x / s)) + z, 0, 255).
//
// Three launches, no atomics and no grid barrier:
//   1. kv_range_kernel: a 512-thread block owns a slab of 512 channels x 320 tokens; each lane
//      loads its 8 channels x 40 tokens in one burst (40 loads in flight), folds min / max,
//      the 8 waves are folded in LDS and the block stores one partial (lo, hi) per channel.
//   2. kv_params_kernel: one thread per channel folds the partials and writes s and z.
//   3. kv_quant_kernel: many small blocks (512 channels x 64 tokens) re-read x -- at the cache
//      sizes of interest it is still in the 256 MB last-level cache -- and write the codes.
// Codes use the correctly rounded quotient fl32(x / s) from one multiply and two FMAs with the
// channel's reciprocal (div_rn), then rne, + z and the clamp: no division per element, no branch.
//
// kv_dequant_kernel writes x' = bf16(fl32((q - z) * s)) (v_cvt_pk_bf16_f32 rounds to nearest
// even) with the quantize pass's tiling.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

constexpr int kKvLanesC = 8;             // channels per lane (one 16-byte bf16 load per row)
constexpr int kKvSlab = 64 * kKvLanesC;  // channels per block (512)
// range pass
constexpr int kRangeWaves = 8;                             // 512 threads: thread t owns channel t
constexpr int kRangeRows = 40;                             // token rows per lane, one burst
constexpr int kRangeTokPerBlock = kRangeWaves * kRangeRows;  // 320
// quantize / dequantize passes
constexpr int kKvWaves = 4;
constexpr int kKvBatch = 16;                               // rows in flight per lane
constexpr int kKvTokPerBlockQ = kKvWaves * kKvBatch;       // 64


// byte k of w as a float (selected to v_cvt_f32_ubyte{k})
__device__ __forceinline__ float byte_to_float(uint32_t w, int k) {
  return (float)((w >> (8 * k)) & 0xFFu);
}

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

// ---------------------------------------------------------------- workspace
// part_lo[chunks][channels], part_hi[chunks][channels]: one partial range per 320-token chunk,
// fully rewritten by every call (no state survives between calls).
__host__ __device__ inline int kv_slabs(int channels) { return (channels + kKvSlab - 1) / kKvSlab; }
__host__ __device__ inline int kv_range_chunks(int tokens) {
  return (tokens + kRangeTokPerBlock - 1) / kRangeTokPerBlock;
}

__device__ __forceinline__ void params_from_range(float lo, float hi, float& s, float& z) {
  s = (hi - lo) / 255.0f;
  if (s == 0.0f) s = 1.0f;
  z = __builtin_fminf(__builtin_fmaxf(rne_quotient(-lo, s, 1.0f / s), 0.0f), 255.0f);
}

// Codes of one row of 8 channels.
__device__ __forceinline__ v2u quant_row8(const v4u w, const float* s, const float* rcp,
                                          const float* z) {
  float v[8];
  decode8_bf16(w, v);
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = rne_quotient(v[i], s[i], rcp[i]) + z[i];
    const float b = rne_quotient(v[4 + i], s[4 + i], rcp[4 + i]) + z[4 + i];
    w0 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(a, 0.0f, 255.0f), i, w0);
    w1 = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(b, 0.0f, 255.0f), i, w1);
  }
  return v2u{w0, w1};
}

__device__ __forceinline__ void load_params8(const float* scale, const uint8_t* zero, int c0,
                                             float* s, float* z) {
  const v4f s0 = reinterpret_cast<const v4f*>(scale + c0)[0];
  const v4f s1 = reinterpret_cast<const v4f*>(scale + c0)[1];
  s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
  s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  const v2u zz = *reinterpret_cast<const v2u*>(zero + c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = byte_to_float(zz.x, i);
    z[4 + i] = byte_to_float(zz.y, i);
  }
}

// ---------------------------------------------------------------- 1. range
__global__ __launch_bounds__(512) void kv_range_kernel(const uint16_t* __restrict__ x, int tokens,
                                                       int channels, float* __restrict__ part_lo,
                                                       float* __restrict__ part_hi) {
  __shared__ float red[2][kRangeWaves][kKvSlab];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // consecutive blocks (which the dispatcher spreads over the XCDs) take consecutive token
  // chunks of one slab
  const int nchunks = gridDim.x / kv_slabs(channels);
  const int slab = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
  const int c0 = slab * kKvSlab + lane * kKvLanesC;
  const int t_begin = chunk * kRangeTokPerBlock + wave * kRangeRows;
  const int nrows = max(0, min(tokens - t_begin, kRangeRows));
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
  if (c0 < channels && nrows > 0) {
    const uint16_t* p = x + (size_t)t_begin * channels + c0;
    v4u rows[kRangeRows];
    if (nrows == kRangeRows) {
#pragma unroll
      for (int b = 0; b < kRangeRows; ++b) rows[b] = *reinterpret_cast<const v4u*>(p + (size_t)b * channels);
    } else {
#pragma unroll
      for (int b = 0; b < kRangeRows; ++b)
        rows[b] = b < nrows ? *reinterpret_cast<const v4u*>(p + (size_t)b * channels) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < kRangeRows; ++b) {
      float v[8];
      decode8_bf16(rows[b], v);  // rows past the end hold +0, which the range already contains
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = __builtin_fminf(lo[i], v[i]);
        hi[i] = __builtin_fmaxf(hi[i], v[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[0][wave][lane * 8 + i] = lo[i];
    red[1][wave][lane * 8 + i] = hi[i];
  }
  __syncthreads();
  float l = 0.0f, h = 0.0f;
#pragma unroll
  for (int w = 0; w < kRangeWaves; ++w) {
    l = __builtin_fminf(l, red[0][w][threadIdx.x]);
    h = __builtin_fmaxf(h, red[1][w][threadIdx.x]);
  }
  const int c = slab * kKvSlab + threadIdx.x;
  if (c < channels) {
    part_lo[(size_t)chunk * channels + c] = l;
    part_hi[(size_t)chunk * channels + c] = h;
  }
}

// ---------------------------------------------------------------- 2. parameters
__global__ __launch_bounds__(256) void kv_params_kernel(const float* __restrict__ part_lo,
                                                        const float* __restrict__ part_hi,
                                                        int nchunks, int channels,
                                                        float* __restrict__ scale,
                                                        uint8_t* __restrict__ zero) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= channels) return;
  float l = 0.0f, h = 0.0f;
  int k = 0;
  for (; k + 8 <= nchunks; k += 8) {  // 8 chunks' loads in flight
    float pl[8], ph[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      pl[b] = part_lo[(size_t)(k + b) * channels + c];
      ph[b] = part_hi[(size_t)(k + b) * channels + c];
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      l = __builtin_fminf(l, pl[b]);
      h = __builtin_fmaxf(h, ph[b]);
    }
  }
  for (; k < nchunks; ++k) {
    l = __builtin_fminf(l, part_lo[(size_t)k * channels + c]);
    h = __builtin_fmaxf(h, part_hi[(size_t)k * channels + c]);
  }
  float s, z;
  params_from_range(l, h, s, z);
  scale[c] = s;
  zero[c] = (uint8_t)z;
}

// ---------------------------------------------------------------- 3. quantize
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ x, int tokens,
                                                       int channels,
                                                       const float* __restrict__ scale,
                                                       const uint8_t* __restrict__ zero,
                                                       uint8_t* __restrict__ q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kKvSlab + lane * kKvLanesC;
  if (c0 >= channels) return;
  const int t_begin = blockIdx.y * kKvTokPerBlockQ + wave * kKvBatch;
  const int t_end = min(tokens, t_begin + kKvBatch);
  float s[8], z[8], rcp[8];
  load_params8(scale, zero, c0, s, z);
#pragma unroll
  for (int i = 0; i < 8; ++i) rcp[i] = 1.0f / s[i];
  const uint16_t* p = x + (size_t)c0;
  uint8_t* d = q + (size_t)c0;
  int t = t_begin;
  for (; t + kKvBatch <= t_end; t += kKvBatch) {
    v4u w[kKvBatch];
#pragma unroll
    for (int b = 0; b < kKvBatch; ++b) w[b] = *reinterpret_cast<const v4u*>(p + (size_t)(t + b) * channels);
#pragma unroll
    for (int b = 0; b < kKvBatch; ++b)
      *reinterpret_cast<v2u*>(d + (size_t)(t + b) * channels) = quant_row8(w[b], s, rcp, z);
  }
  for (; t < t_end; ++t)
    *reinterpret_cast<v2u*>(d + (size_t)t * channels) =
        quant_row8(*reinterpret_cast<const v4u*>(p + (size_t)t * channels), s, rcp, z);
}

__global__ __launch_bounds__(256) void kv_dequant_kernel(const uint8_t* __restrict__ q,
                                                         const float* __restrict__ scale,
                                                         const uint8_t* __restrict__ zero,
                                                         int tokens, int channels,
                                                         uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kKvSlab + lane * kKvLanesC;
  if (c0 >= channels) return;
  const int t_begin = blockIdx.y * kKvTokPerBlockQ + wave * kKvBatch;
  const int t_end = min(tokens, t_begin + kKvBatch);
  float s[8], z[8];
  load_params8(scale, zero, c0, s, z);
  const uint8_t* p = q + (size_t)c0;
  uint16_t* d = out + (size_t)c0;
  auto dequant_row = [&](const v2u w) -> v4u {
    float c[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = byte_to_float(w.x, i);
      c[4 + i] = byte_to_float(w.y, i);
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (q - z) is a small exact integer; one rounding for the product, one for bf16
      const v2f pr = v2f{(c[2 * i] - z[2 * i]) * s[2 * i], (c[2 * i + 1] - z[2 * i + 1]) * s[2 * i + 1]};
      o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, v2bf));
    }
    return v4u{o[0], o[1], o[2], o[3]};
  };
  int t = t_begin;
  for (; t + kKvBatch <= t_end; t += kKvBatch) {
    v2u w[kKvBatch];
#pragma unroll
    for (int b = 0; b < kKvBatch; ++b) w[b] = *reinterpret_cast<const v2u*>(p + (size_t)(t + b) * channels);
#pragma unroll
    for (int b = 0; b < kKvBatch; ++b) *reinterpret_cast<v4u*>(d + (size_t)(t + b) * channels) = dequant_row(w[b]);
  }
  for (; t < t_end; ++t)
    *reinterpret_cast<v4u*>(d + (size_t)t * channels) = dequant_row(*reinterpret_cast<const v2u*>(p + (size_t)t * channels));
}

// ---------------------------------------------------------------- host side
size_t kv_workspace_bytes(int tokens, int channels) {
  if (tokens <= 0 || channels <= 0) return 0;
  return (size_t)2 * kv_range_chunks(tokens) * channels * sizeof(float);
}

hipError_t launch_kv_quant(const uint16_t* x, int tokens, int channels, uint8_t* q,
                           float* scale, uint8_t* zero, void* workspace, hipStream_t stream) {
  const int nslabs = kv_slabs(channels), nchunks = kv_range_chunks(tokens);
  float* part_lo = reinterpret_cast<float*>(workspace);
  float* part_hi = part_lo + (size_t)nchunks * channels;
  hipLaunchKernelGGL(kv_range_kernel, dim3(nslabs * nchunks), dim3(512), 0, stream, x, tokens,
                     channels, part_lo, part_hi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_params_kernel, dim3((channels + 255) / 256), dim3(256), 0, stream, part_lo,
                     part_hi, nchunks, channels, scale, zero);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid_q(nslabs, (tokens + kKvTokPerBlockQ - 1) / kKvTokPerBlockQ);
  hipLaunchKernelGGL(kv_quant_kernel, grid_q, dim3(256), 0, stream, x, tokens, channels, scale,
                     zero, q);
  return hipGetLastError();
}

hipError_t launch_kv_dequant(const uint8_t* q, const float* scale, const uint8_t* zero,
                             int tokens, int channels, uint16_t* x_out, hipStream_t stream) {
  const dim3 grid(kv_slabs(channels), (tokens + kKvTokPerBlockQ - 1) / kKvTokPerBlockQ);
  hipLaunchKernelGGL(kv_dequant_kernel, grid, dim3(256), 0, stream, q, scale, zero, tokens,
                     channels, x_out);
  return hipGetLastError();
}

}  // namespace svdq
