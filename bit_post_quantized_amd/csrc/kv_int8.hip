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
// Two schedules compute the same codes:
//  * the fused single pass (kv_quant_fused_kernel, below) reads x from HBM once and keeps it in
//    registers while the blocks that share a 128-channel slab agree on its range through the
//    workspace.  It runs when channels are a multiple of 128, an eighth of the tokens fits in
//    40 rows per thread, and the device holds the whole grid at once.
//  * otherwise three launches, no atomics and no grid barrier:
//   1. kv_range_kernel: a block owns 512 channels x 64 tokens (the blocks of one token chunk
//      are grid neighbours, so the pass streams whole rows); each lane loads its 8 channels x 16
//      tokens in one burst, folds min / max, the 4 waves are folded in LDS and the block stores
//      one partial (lo, hi) per channel.
//   2. kv_params_kernel: 8 threads per channel fold the partials, meet in LDS, and write s, z.
//   3. kv_quant_kernel: many small blocks (512 channels x 64 tokens) re-read x and write the
//      codes.
// Codes use the correctly rounded quotient fl32(x / s) from one multiply and two FMAs with the
// channel's reciprocal (div_rn), then rne, + z and the clamp: no division per element, no branch.
//
// kv_dequant_kernel writes x' = bf16(fl32((q - z) * s)) (v_cvt_pk_bf16_f32 rounds to nearest
// even): blocks of 512 channels x 32 tokens, each lane 8 channels of 8 rows.
//
// The fused pass and the dequantization touch each byte once: their loads and stores are
// non-temporal, so the streams pass the caches without displacing other data.  A plain read
// stream that follows a large write (another tensor's dequantization, a GEMM's output) evicts
// those dirty lines and waits on their write-back; 84 MB of x then took 47 us instead of 32.
#include <atomic>
#include <chrono>
#include <cstdlib>

#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

constexpr int kKvLanesC = 8;             // channels per lane (one 16-byte bf16 load per row)
constexpr int kKvSlab = 64 * kKvLanesC;  // channels per block (512)
// every pass: a block of 4 waves covers 512 channels x 64 tokens; lane l of wave w owns 8
// channels (one 16-byte bf16 load per row) of the wave's 16 rows, all 16 loads in flight
constexpr int kKvWaves = 4;
constexpr int kKvBatch = 16;                               // rows in flight per lane
constexpr int kKvTokPerBlockQ = kKvWaves * kKvBatch;       // 64
constexpr int kRangeTokPerBlock = kKvTokPerBlockQ;         // one partial range per 64 tokens
// dequantization: 8 rows in flight per lane, so a block covers 512 channels x 32 tokens (16
// rows per lane and 64 tokens per block took 26.1 against 24.9 us per tensor in the bench step;
// 32 rows 30.4)
constexpr int kDeqBatch = 8;
constexpr int kDeqTokPerBlock = kKvWaves * kDeqBatch;      // 32
// parameter fold: a block of 256 threads folds 32 channels; 8 threads per channel split the chunks
constexpr int kFoldChannels = 32;
constexpr int kFoldSplit = 8;


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
// part_lo[chunks][channels], part_hi[chunks][channels]: one partial range per 64-token chunk,
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
// Grid (slab, chunk) with the slab fastest: the 8 blocks that cover one 64-token chunk of all
// channels are neighbours, so the pass streams whole rows.
__global__ __launch_bounds__(256) void kv_range_kernel(const uint16_t* __restrict__ x, int tokens,
                                                       int channels, float* __restrict__ part_lo,
                                                       float* __restrict__ part_hi) {
  __shared__ float red[2][kKvWaves][kKvSlab];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kKvSlab + lane * kKvLanesC;
  const int chunk = blockIdx.y;
  const int t_begin = chunk * kRangeTokPerBlock + wave * kKvBatch;
  const int nrows = max(0, min(tokens - t_begin, kKvBatch));
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
  if (c0 < channels && nrows > 0) {
    const uint16_t* p = x + (size_t)t_begin * channels + c0;
    v4u rows[kKvBatch];
    if (nrows == kKvBatch) {
#pragma unroll
      for (int b = 0; b < kKvBatch; ++b) rows[b] = *reinterpret_cast<const v4u*>(p + (size_t)b * channels);
    } else {
      // tail chunk: re-read the last valid row (its values are already in the range)
#pragma unroll
      for (int b = 0; b < kKvBatch; ++b)
        rows[b] = *reinterpret_cast<const v4u*>(p + (size_t)min(b, nrows - 1) * channels);
    }
#pragma unroll
    for (int b = 0; b < kKvBatch; ++b) {
      float v[8];
      decode8_bf16(rows[b], v);
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
  // thread t folds the 4 waves for channels t and t + 256 of the slab
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cl = threadIdx.x + 256 * h;
    float l = 0.0f, u = 0.0f;
#pragma unroll
    for (int w = 0; w < kKvWaves; ++w) {
      l = __builtin_fminf(l, red[0][w][cl]);
      u = __builtin_fmaxf(u, red[1][w][cl]);
    }
    const int c = blockIdx.x * kKvSlab + cl;
    if (c < channels) {
      part_lo[(size_t)chunk * channels + c] = l;
      part_hi[(size_t)chunk * channels + c] = u;
    }
  }
}

// ---------------------------------------------------------------- 2. parameters
// A block folds the partial ranges of 32 channels: thread (j, c) folds chunks j, j + 8, ... of
// channel c (coalesced over c), then the 8 partial folds meet in LDS.
__global__ __launch_bounds__(256) void kv_params_kernel(const float* __restrict__ part_lo,
                                                        const float* __restrict__ part_hi,
                                                        int nchunks, int channels,
                                                        float* __restrict__ scale,
                                                        uint8_t* __restrict__ zero) {
  __shared__ float red[2][kFoldSplit][kFoldChannels];
  const int cl = threadIdx.x % kFoldChannels, j = threadIdx.x / kFoldChannels;
  const int c = blockIdx.x * kFoldChannels + cl;
  const int cc = min(c, channels - 1);
  float l = 0.0f, h = 0.0f;
  int k = j;
  for (; k + 3 * kFoldSplit < nchunks; k += 4 * kFoldSplit) {  // 4 chunks' loads in flight
    float pl[4], ph[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      pl[b] = part_lo[(size_t)(k + b * kFoldSplit) * channels + cc];
      ph[b] = part_hi[(size_t)(k + b * kFoldSplit) * channels + cc];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      l = __builtin_fminf(l, pl[b]);
      h = __builtin_fmaxf(h, ph[b]);
    }
  }
  for (; k < nchunks; k += kFoldSplit) {
    l = __builtin_fminf(l, part_lo[(size_t)k * channels + cc]);
    h = __builtin_fmaxf(h, part_hi[(size_t)k * channels + cc]);
  }
  red[0][j][cl] = l;
  red[1][j][cl] = h;
  __syncthreads();
  if (j == 0 && c < channels) {
#pragma unroll
    for (int w = 1; w < kFoldSplit; ++w) {
      l = __builtin_fminf(l, red[0][w][cl]);
      h = __builtin_fmaxf(h, red[1][w][cl]);
    }
    float s, z;
    params_from_range(l, h, s, z);
    scale[c] = s;
    zero[c] = (uint8_t)z;
  }
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
  const int t_begin = blockIdx.y * kDeqTokPerBlock + wave * kDeqBatch;
  const int t_end = min(tokens, t_begin + kDeqBatch);
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
  for (; t + kDeqBatch <= t_end; t += kDeqBatch) {
    v2u w[kDeqBatch];
#pragma unroll
    for (int b = 0; b < kDeqBatch; ++b) w[b] = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p + (size_t)(t + b) * channels));
#pragma unroll
    for (int b = 0; b < kDeqBatch; ++b) __builtin_nontemporal_store(dequant_row(w[b]), reinterpret_cast<v4u*>(d + (size_t)(t + b) * channels));
  }
  for (; t < t_end; ++t)
    *reinterpret_cast<v4u*>(d + (size_t)t * channels) = dequant_row(*reinterpret_cast<const v2u*>(p + (size_t)t * channels));
}

// ---------------------------------------------------------------- fused single pass
// x is read from HBM once: a block keeps its share of x in registers while the per-channel
// range is agreed, then codes it from registers.  A slab of 128 channels (256 bytes of a bf16
// row, one whole 128-byte line of its codes) is split over kFusedParts blocks by tokens (a
// 64-channel slab writes half lines, which two XCDs then write back separately, and loads
// 128-byte strips; both measured slower); each block folds min / max over its
// tokens, publishes the partial range in the workspace with the call's epoch as a tag, waits
// for the other parts' tags, folds the parts, and quantizes.  The parts of a slab are mapped
// to blocks that the dispatcher places on one XCD (block b runs on XCD b % 8), so the exchange
// mostly stays in one L2.  The wait is bounded: a block that times out (e.g. when not every
// part of its slab is resident) computes the slab's range from x itself, so the result never
// depends on the exchange and the kernel always finishes.
constexpr int kFusedCh = 128;
constexpr int kFusedParts = 8;
constexpr int kFusedThreads = 512;
constexpr int kFusedRowThreads = kFusedCh / kKvLanesC;                // 16 threads share a row
constexpr int kFusedRowsPerPass = kFusedThreads / kFusedRowThreads;   // 32 rows per pass
constexpr int kFusedMaxRows = 40;                                     // rows per thread
constexpr int kFusedSegs = kFusedThreads / kFusedCh;                  // 4 fold segments of 8 rows
static_assert(kFusedSegs * 8 == kFusedRowsPerPass, "block fold: segments of 8 rows");
constexpr int kFusedInFlight = 8;                                     // row loads in flight

__device__ __forceinline__ void fused_slab_part(int b, int nslabs, int& slab, int& part) {
  if (nslabs % 8 == 0) {  // the kFusedParts blocks of a slab share XCD b % 8
    const int xcd = b & 7, j = b >> 3;
    part = j % kFusedParts;
    slab = (j / kFusedParts) * 8 + xcd;
  } else {
    slab = b / kFusedParts;
    part = b % kFusedParts;
  }
}

template <int R>  // token rows per thread held in registers
__global__ __launch_bounds__(kFusedThreads) void kv_quant_fused_kernel(
    const uint16_t* __restrict__ x, int tokens, int channels, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint8_t* __restrict__ zero, uint32_t* __restrict__ tags,
    float* __restrict__ parts, uint32_t epoch, long long spin_ticks) {
  __shared__ float red[2][kFusedSegs][kFusedCh];
  __shared__ float prm[3][kFusedCh];  // s, 1 / s, z
  __shared__ int fallback;
  const int nslabs = channels / kFusedCh;
  int slab, part;
  fused_slab_part(blockIdx.x, nslabs, slab, part);
  const int tid = threadIdx.x;
  const int lc = tid % kFusedRowThreads, rr = tid / kFusedRowThreads;
  const int c0 = slab * kFusedCh + lc * kKvLanesC;
  const int per = (tokens + kFusedParts - 1) / kFusedParts;
  const int t0 = part * per, t1 = min(tokens, t0 + per);

  // ---- load this thread's rows (row index clamped into the tensor: a duplicate row leaves
  //      min / max unchanged) and fold min / max of its 8 channels
  // At most kFusedInFlight rows of a thread are in flight: with every row of the grid requested
  // at once the memory system serves some waves far later than the others, and every block
  // waits for the slowest part of its slab.
  v4u v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int t = min(t0 + rr + kFusedRowsPerPass * k, tokens - 1);
    v[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + (size_t)t * channels + c0));
    if (k >= kFusedInFlight) asm volatile("" : "+v"(v[k - kFusedInFlight])::"memory");
  }
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    float f[8];
    decode8_bf16(v[k], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = __builtin_fminf(lo[i], f[i]);
      hi[i] = __builtin_fmaxf(hi[i], f[i]);
    }
  }
  // block fold: kFusedRowsPerPass row-threads per channel -> segments of 8 rows in LDS -> 1
  auto block_fold = [&](float* out_lo, float* out_hi) {
    __shared__ float stage[2][kFusedRowsPerPass][kFusedCh + 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      stage[0][rr][lc * 8 + i] = lo[i];
      stage[1][rr][lc * 8 + i] = hi[i];
    }
    __syncthreads();
    {
      const int ch = tid % kFusedCh, seg = tid / kFusedCh;  // segments of 8 rows
      float l = 0.0f, h = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        l = __builtin_fminf(l, stage[0][seg * 8 + k][ch]);
        h = __builtin_fmaxf(h, stage[1][seg * 8 + k][ch]);
      }
      red[0][seg][ch] = l;
      red[1][seg][ch] = h;
    }
    __syncthreads();
    if (tid < kFusedCh) {
      float l = 0.0f, h = 0.0f;
#pragma unroll
      for (int k = 0; k < kFusedSegs; ++k) {
        l = __builtin_fminf(l, red[0][k][tid]);
        h = __builtin_fmaxf(h, red[1][k][tid]);
      }
      *out_lo = l;
      *out_hi = h;
    }
  };
  float plo = 0.0f, phi = 0.0f;
  block_fold(&plo, &phi);
  // keep only the packed rows live across the exchange (the codes decode them again)
#pragma unroll
  for (int k = 0; k < R; ++k) asm volatile("" : "+v"(v[k]));

  // ---- publish this part's range, then wait (bounded) for the other parts
  float* mine = parts + ((size_t)slab * kFusedParts + part) * 2 * kFusedCh;
  if (tid < kFusedCh) {
    mine[tid] = plo;
    mine[kFusedCh + tid] = phi;
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: lane p < kFusedParts watches part p's tag
    if (tid == 0)
      __hip_atomic_store(tags + slab * kFusedParts + part, epoch, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    int fb = 0;
    const long long start = wall_clock64();
    // relaxed polling of all the tags at once, one round trip per poll (an acquire per poll
    // would invalidate caches on every iteration; tags polled one after the other cost one
    // round trip each: 4.8 us from the slowest part's publication to the exchange's end);
    // the acquire fence after the wait orders the reads of the partial ranges
    for (;;) {
      const bool seen = tid >= kFusedParts ||
                        __hip_atomic_load(tags + slab * kFusedParts + tid, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == epoch;
      if (__all(seen)) break;  // uniform over the wave
      if (wall_clock64() - start > spin_ticks) {
        fb = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    // one acquire (it invalidates the CU's vector cache, which every wave shares) before the
    // barrier after which the partial ranges are read
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) fallback = fb;
  }
  __syncthreads();
  if (!fallback) {
    if (tid < kFusedCh) {
      float l = 0.0f, h = 0.0f;
      const float* all = parts + (size_t)slab * kFusedParts * 2 * kFusedCh;
#pragma unroll
      for (int p = 0; p < kFusedParts; ++p) {
        l = __builtin_fminf(l, __hip_atomic_load(all + p * 2 * kFusedCh + tid, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
        h = __builtin_fmaxf(h, __hip_atomic_load(all + p * 2 * kFusedCh + kFusedCh + tid,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      plo = l;
      phi = h;
    }
  } else {
    // the slab's range straight from x: every token, one pass of rows after the other
#pragma unroll
    for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
    for (int t = rr; t < tokens; t += kFusedRowsPerPass) {
      float f[8];
      decode8_bf16(*reinterpret_cast<const v4u*>(x + (size_t)t * channels + c0), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = __builtin_fminf(lo[i], f[i]);
        hi[i] = __builtin_fmaxf(hi[i], f[i]);
      }
    }
    block_fold(&plo, &phi);
  }
  if (tid < kFusedCh) {
    float s, z;
    params_from_range(plo, phi, s, z);
    prm[0][tid] = s;
    prm[1][tid] = 1.0f / s;
    prm[2][tid] = z;
    if (part == 0) {
      scale[slab * kFusedCh + tid] = s;
      zero[slab * kFusedCh + tid] = (uint8_t)z;
    }
  }
  __syncthreads();

  // ---- codes of the resident rows
  float s8[8], r8[8], z8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s8[i] = prm[0][lc * 8 + i];
    r8[i] = prm[1][lc * 8 + i];
    z8[i] = prm[2][lc * 8 + i];
  }
  // Rows t0 + rr + 64 k, k < nk, are this thread's: one live count and one moving pointer.  (A
  // token index per row does not fit beside the rows; a spilled one costs a wait on every row,
  // because stores count in the same counter as the spill reload.)
  const int nk = max(0, (t1 - t0 - rr + kFusedRowsPerPass - 1) / kFusedRowsPerPass);
  uint8_t* qp = q + (size_t)(t0 + rr) * channels + c0;
  const size_t pass = (size_t)kFusedRowsPerPass * channels;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < nk) __builtin_nontemporal_store(quant_row8(v[k], s8, r8, z8), reinterpret_cast<v2u*>(qp));
    qp += pass;
  }
}

// ---------------------------------------------------------------- host side
static int fused_rows(int tokens, int channels) {
  if (channels % kFusedCh != 0 || tokens <= 0) return 0;
  const int per = (tokens + kFusedParts - 1) / kFusedParts;
  const int rows = (per + kFusedRowsPerPass - 1) / kFusedRowsPerPass;
  return rows <= kFusedMaxRows ? rows : 0;
}

size_t kv_workspace_bytes(int tokens, int channels) {
  if (tokens <= 0 || channels <= 0) return 0;
  const size_t three_pass = (size_t)2 * kv_range_chunks(tokens) * channels * sizeof(float);
  const size_t nslabs = (size_t)(channels / kFusedCh);
  const size_t fused = nslabs * kFusedParts * (16 + 2 * kFusedCh * sizeof(float));
  return three_pass > fused ? three_pass : fused;
}

// Epoch of a fused call: strictly increasing per process, started at a time-dependent value,
// so a tag left in a workspace by an earlier call (or by whatever the memory held before)
// never matches the running call.
static uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
  uint32_t e = counter.fetch_add(1) + 1;
  return e ? e : counter.fetch_add(1) + 1;
}

// Spin limit of the fused pass's exchange, in 100 MHz wall-clock ticks (default 100 ms; the
// variable SVDQ_KV_SPIN_TICKS overrides it -- 0 forces every block down the self-contained path).
static long long spin_ticks() {
  const char* v = std::getenv("SVDQ_KV_SPIN_TICKS");
  return v ? std::atoll(v) : 10000000LL;
}

// Blocks of kv_quant_fused_kernel<8 n> that the current device holds at once (0 if unknown).
// The exchange waits for every part of a slab, so the fused pass is launched only when the
// whole grid is resident together; the bounded wait stays as the guard for anything else
// sharing the device.
static int fused_resident_blocks(int n) {
  static const void* const fns[6] = {
      nullptr,
      reinterpret_cast<const void*>(&kv_quant_fused_kernel<8>),
      reinterpret_cast<const void*>(&kv_quant_fused_kernel<16>),
      reinterpret_cast<const void*>(&kv_quant_fused_kernel<24>),
      reinterpret_cast<const void*>(&kv_quant_fused_kernel<32>),
      reinterpret_cast<const void*>(&kv_quant_fused_kernel<40>)};
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][6];  // value + 1; 0 = not yet queried
  int dev = 0;
  if (n < 1 || n > 5 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int c = cache[dev][n].load(std::memory_order_relaxed);
  if (c) return c - 1;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fns[n], kFusedThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error behind; use the three-pass path
    return 0;
  }
  const int blocks = per_cu * cus;
  cache[dev][n].store(blocks + 1, std::memory_order_relaxed);
  return blocks;
}

hipError_t launch_kv_quant(const uint16_t* x, int tokens, int channels, uint8_t* q,
                           float* scale, uint8_t* zero, void* workspace, hipStream_t stream) {
  const int rows = fused_rows(tokens, channels);
  if (rows > 0 && (channels / kFusedCh) * kFusedParts <= fused_resident_blocks((rows + 7) / 8)) {
    const int nslabs = channels / kFusedCh;
    uint32_t* tags = reinterpret_cast<uint32_t*>(workspace);
    float* parts = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                            (size_t)nslabs * kFusedParts * 16);
    const dim3 grid(nslabs * kFusedParts), block(kFusedThreads);
    const uint32_t epoch = next_epoch();
    const long long ticks = spin_ticks();
    switch ((rows + 7) / 8) {
#define SVDQ_KV_FUSED(n)                                                                       \
  case n:                                                                                      \
    hipLaunchKernelGGL(kv_quant_fused_kernel<8 * n>, grid, block, 0, stream, x, tokens,        \
                       channels, q, scale, zero, tags, parts, epoch, ticks);                   \
    break;
      SVDQ_KV_FUSED(1)
      SVDQ_KV_FUSED(2)
      SVDQ_KV_FUSED(3)
      SVDQ_KV_FUSED(4)
      SVDQ_KV_FUSED(5)
#undef SVDQ_KV_FUSED
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int nslabs = kv_slabs(channels), nchunks = kv_range_chunks(tokens);
  float* part_lo = reinterpret_cast<float*>(workspace);
  float* part_hi = part_lo + (size_t)nchunks * channels;
  hipLaunchKernelGGL(kv_range_kernel, dim3(nslabs, nchunks), dim3(256), 0, stream, x, tokens,
                     channels, part_lo, part_hi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_params_kernel, dim3((channels + kFoldChannels - 1) / kFoldChannels),
                     dim3(256), 0, stream, part_lo, part_hi, nchunks, channels, scale, zero);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid_q(nslabs, (tokens + kKvTokPerBlockQ - 1) / kKvTokPerBlockQ);
  hipLaunchKernelGGL(kv_quant_kernel, grid_q, dim3(256), 0, stream, x, tokens, channels, scale,
                     zero, q);
  return hipGetLastError();
}

hipError_t launch_kv_dequant(const uint8_t* q, const float* scale, const uint8_t* zero,
                             int tokens, int channels, uint16_t* x_out, hipStream_t stream) {
  const dim3 grid(kv_slabs(channels), (tokens + kDeqTokPerBlock - 1) / kDeqTokPerBlock);
  hipLaunchKernelGGL(kv_dequant_kernel, grid, dim3(256), 0, stream, q, scale, zero, tokens,
                     channels, x_out);
  return hipGetLastError();
}

}  // namespace svdq
