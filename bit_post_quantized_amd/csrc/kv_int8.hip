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
#include <mutex>

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

// Range of 8 channels folded on the raw bf16 bits, two channels per packed 16-bit max.  A
// non-negative bf16's bits order as a signed 16-bit integer and every negative one compares
// below them, so the signed max over a channel (from 0) is the bits of max(0, max x); a
// negative bf16's bits order by magnitude as an unsigned 16-bit integer and compare above every
// non-negative one, so the unsigned max (from 0) has its sign bit set exactly when the channel
// holds a negative value, and is then the bits of min x.  (x is finite.)
typedef short v2s16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2s16, a),
                                                                __builtin_bit_cast(v2s16, b)));
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16, a),
                                                                __builtin_bit_cast(v2u16, b)));
}

// hb, lb: the signed and unsigned packed maxima of 8 channels (channel 2j in the low half of
// word j) -> lo = min(0, min x), hi = max(0, max x) as floats
__device__ __forceinline__ void range_from_bits(const uint32_t* hb, const uint32_t* lb,
                                                float* lo, float* hi) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[2 * j] = __uint_as_float(hb[j] << 16);
    hi[2 * j + 1] = __uint_as_float(hb[j] & 0xFFFF0000u);
    lo[2 * j] = (lb[j] & 0x8000u) ? __uint_as_float(lb[j] << 16) : 0.0f;
    lo[2 * j + 1] = (lb[j] & 0x80000000u) ? __uint_as_float(lb[j] & 0xFFFF0000u) : 0.0f;
  }
}

// ---------------------------------------------------------------- workspace
// part_lo[chunks][channels], part_hi[chunks][channels]: one partial range per 64-token chunk,
// fully rewritten by every call (no state survives between calls).
// (counts of a positive int, rounded up, in 64-bit arithmetic so no int overflows)
__host__ __device__ inline int kv_slabs(int channels) {
  return (int)(((long long)channels + kKvSlab - 1) / kKvSlab);
}
__host__ __device__ inline int kv_range_chunks(int tokens) {
  return (int)(((long long)tokens + kRangeTokPerBlock - 1) / kRangeTokPerBlock);
}

__device__ __forceinline__ void params_from_range(float lo, float hi, float& s, float& z) {
  s = (hi - lo) / 255.0f;
  if (s == 0.0f) s = 1.0f;
  z = __builtin_fminf(__builtin_fmaxf(rne_quotient(-lo, s, 1.0f / s), 0.0f), 255.0f);
}

// Codes of one row of 8 channels.  rne(x / s) + z is an integer in fp32; v_cvt_pk_u8_f32
// converts it exactly and saturates to [0, 255], which is the clamp.
__device__ __forceinline__ v2u quant_row8(const v4u w, const float* s, const float* rcp,
                                          const float* z) {
  float v[8];
  decode8_bf16(w, v);
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 = __builtin_amdgcn_cvt_pk_u8_f32(rne_quotient(v[i], s[i], rcp[i]) + z[i], i, w0);
    w1 = __builtin_amdgcn_cvt_pk_u8_f32(rne_quotient(v[4 + i], s[4 + i], rcp[4 + i]) + z[4 + i],
                                        i, w1);
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
// 128-byte strips; both measured slower); each block folds min / max over its tokens,
// publishes the partial range in the workspace, reads the other parts' ranges, folds them, and
// quantizes.  The parts of a slab are mapped to blocks that the dispatcher places on one XCD
// (block b runs on XCD b % 8).
//
// The exchange needs no fence.  Every published word is one 64-bit relaxed atomic store at
// agent scope holding (call epoch, float bits); a reader accepts a word only when it carries
// the running call's epoch.  Each word is validated by itself (a single location is coherent,
// and a 64-bit atomic is never seen torn), so no ordering between words, waves or blocks is
// needed.  (The first design published plain stores behind release fences; on this device an
// agent-scope release writes back the XCD's L2, which took 6.5 to 9 us per exchange out of a
// 30 us call.)  The wait is bounded: a block whose wait times out (e.g. when not every part of
// its slab is resident) computes the slab's range from x itself, so the result never depends
// on the exchange and the kernel always finishes.
//
// The paired form quantizes two tensors of one shape (a layer's K and V) in one launch: once a
// block has the first tensor's parameters it stores each row's codes and loads the second
// tensor's row into the registers that row held; then the second tensor's range is agreed and
// its codes written as in the single form.
constexpr int kFusedCh = 128;
constexpr int kFusedParts = 8;
constexpr int kFusedThreads = 512;
constexpr int kFusedRowThreads = kFusedCh / kKvLanesC;                // 16 threads share a row
constexpr int kFusedRowsPerPass = kFusedThreads / kFusedRowThreads;   // 32 rows per pass
constexpr int kFusedMaxRows = 40;                                     // rows per thread
constexpr int kFusedSegs = kFusedThreads / kFusedCh;                  // 4 fold segments of 8 rows
static_assert(kFusedSegs * 8 == kFusedRowsPerPass, "block fold: segments of 8 rows");
constexpr int kFusedInFlight = 8;                                     // row loads in flight
// row loads in flight while the paired form stores the first tensor's codes (the stores count
// in the same in-order counter as the loads, so a wait for a load also waits for every store
// issued before it)
constexpr int kPairInFlight = 8;
// workspace of one tensor: per part of a slab, 2 x 128 words (lo, hi) of (epoch << 32 | bits)
constexpr size_t kFusedPartBytes = 2 * kFusedCh * sizeof(uint64_t);

__host__ __device__ inline size_t fused_region_bytes(int channels) {
  return (size_t)(channels / kFusedCh) * kFusedParts * kFusedPartBytes;
}

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

// One tensor of a fused call: its rows, outputs, and its region of the workspace (the parts'
// published partial ranges, [slab][part][lo 128 | hi 128] words).
struct KvFusedTensor {
  const uint16_t* x;
  uint8_t* q;
  float* scale;
  uint8_t* zero;
  uint64_t* parts;
};

struct KvFusedShared {
  float stage[2][kFusedRowsPerPass][kFusedCh + 1];
  float red[2][kFusedSegs][kFusedCh];
  float prm[3][kFusedCh];  // s, 1 / s, z of the slab's channels
};

// Block-wide min / max of the slab's channels over this block's rows: thread (rr, lc) holds the
// range of its 8 channels over its rows; on return threads 0..127 hold channel tid's range.
__device__ __forceinline__ void fused_block_fold(KvFusedShared& sh, const float* lo,
                                                 const float* hi, float& out_lo, float& out_hi) {
  const int tid = threadIdx.x;
  const int lc = tid % kFusedRowThreads, rr = tid / kFusedRowThreads;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sh.stage[0][rr][lc * 8 + i] = lo[i];
    sh.stage[1][rr][lc * 8 + i] = hi[i];
  }
  __syncthreads();
  {
    const int ch = tid % kFusedCh, seg = tid / kFusedCh;  // segments of 8 rows
    float l = 0.0f, h = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      l = __builtin_fminf(l, sh.stage[0][seg * 8 + k][ch]);
      h = __builtin_fmaxf(h, sh.stage[1][seg * 8 + k][ch]);
    }
    sh.red[0][seg][ch] = l;
    sh.red[1][seg][ch] = h;
  }
  __syncthreads();
  if (tid < kFusedCh) {
    float l = 0.0f, h = 0.0f;
#pragma unroll
    for (int k = 0; k < kFusedSegs; ++k) {
      l = __builtin_fminf(l, sh.red[0][k][tid]);
      h = __builtin_fmaxf(h, sh.red[1][k][tid]);
    }
    out_lo = l;
    out_hi = h;
  }
}

__device__ __forceinline__ uint64_t tagged(uint32_t epoch, float v) {
  return ((uint64_t)epoch << 32) | __float_as_uint(v);
}

// From this block's folded range (lo / hi of the thread's 8 channels) to the slab's parameters
// in sh.prm: publish the part's range, read every part's range once it carries this call's
// epoch (bounded wait), fold them; on a time-out, the slab's range straight from x.  Part 0
// stores the slab's scale and zero.
__device__ __forceinline__ void fused_slab_params(KvFusedShared& sh, const KvFusedTensor& T,
                                               float* lo, float* hi, int tokens, int channels,
                                               int slab, int part, uint32_t epoch,
                                               long long spin_ticks) {
  const int tid = threadIdx.x;
  const int lc = tid % kFusedRowThreads, rr = tid / kFusedRowThreads;
  const int c0 = slab * kFusedCh + lc * kKvLanesC;
  float plo = 0.0f, phi = 0.0f;
  fused_block_fold(sh, lo, hi, plo, phi);

  int timed_out = 0;
  if (tid < kFusedCh) {  // thread tid owns channel tid of the slab: waves 0 and 1
    uint64_t* all = T.parts + (size_t)slab * kFusedParts * 2 * kFusedCh;
    uint64_t* mine = all + (size_t)part * 2 * kFusedCh;
    __hip_atomic_store(mine + tid, tagged(epoch, plo), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + kFusedCh + tid, tagged(epoch, phi), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    // every part's (lo, hi) of channel tid, 16 loads per poll; parts already seen are kept
    uint64_t w[2 * kFusedParts];
    uint32_t pending = (1u << (2 * kFusedParts)) - 1u;
    const long long start = wall_clock64();
    for (;;) {
#pragma unroll
      for (int i = 0; i < 2 * kFusedParts; ++i)
        if (pending & (1u << i))
          w[i] = __hip_atomic_load(all + (size_t)(i >> 1) * 2 * kFusedCh + (i & 1) * kFusedCh + tid,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < 2 * kFusedParts; ++i)
        if ((uint32_t)(w[i] >> 32) == epoch) pending &= ~(1u << i);
      if (pending == 0u) break;
      if (wall_clock64() - start > spin_ticks) {
        timed_out = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!timed_out) {
      float l = 0.0f, h = 0.0f;
#pragma unroll
      for (int p = 0; p < kFusedParts; ++p) {
        l = __builtin_fminf(l, __uint_as_float((uint32_t)w[2 * p]));
        h = __builtin_fmaxf(h, __uint_as_float((uint32_t)w[2 * p + 1]));
      }
      plo = l;
      phi = h;
    }
  }
  if (__syncthreads_or(timed_out)) {
    // the slab's range straight from x: every token, one pass of rows after the other
#pragma unroll
    for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0.0f;
    for (int t = rr; t < tokens; t += kFusedRowsPerPass) {
      float f[8];
      decode8_bf16(*reinterpret_cast<const v4u*>(T.x + (size_t)t * channels + c0), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = __builtin_fminf(lo[i], f[i]);
        hi[i] = __builtin_fmaxf(hi[i], f[i]);
      }
    }
    fused_block_fold(sh, lo, hi, plo, phi);
  }
  if (tid < kFusedCh) {
    float s, z;
    params_from_range(plo, phi, s, z);
    sh.prm[0][tid] = s;
    sh.prm[1][tid] = 1.0f / s;
    sh.prm[2][tid] = z;
    if (part == 0) {
      T.scale[slab * kFusedCh + tid] = s;
      T.zero[slab * kFusedCh + tid] = (uint8_t)z;
    }
  }
  __syncthreads();
}

template <int R, bool kPair>  // token rows per thread held in registers; two tensors or one
__global__ __launch_bounds__(kFusedThreads) void kv_quant_fused_kernel(
    KvFusedTensor a, KvFusedTensor b, int tokens, int channels, uint32_t epoch,
    long long spin_ticks) {
  __shared__ KvFusedShared sh;
  const int nslabs = channels / kFusedCh;
  int slab, part;
  fused_slab_part(blockIdx.x, nslabs, slab, part);
  const int tid = threadIdx.x;
  const int lc = tid % kFusedRowThreads, rr = tid / kFusedRowThreads;
  const int c0 = slab * kFusedCh + lc * kKvLanesC;
  const int per = (tokens + kFusedParts - 1) / kFusedParts;
  const int t0 = part * per, t1 = min(tokens, t0 + per);
  // Rows t0 + rr + 32 k, k < nk, are this thread's: one live count and one moving pointer per
  // stream.  (A token index per row does not fit beside the rows; a spilled one costs a wait on
  // every row, because stores count in the same counter as the spill reload.)  Loads clamp the
  // row index into the tensor: a duplicate row leaves min / max unchanged.
  const int nk = max(0, (t1 - t0 - rr + kFusedRowsPerPass - 1) / kFusedRowsPerPass);
  const size_t pass = (size_t)kFusedRowsPerPass * channels;
  auto row_of = [&](const uint16_t* x, int k) {
    return reinterpret_cast<const v4u*>(
        x + (size_t)min(t0 + rr + kFusedRowsPerPass * k, tokens - 1) * channels + c0);
  };

  // ---- load this thread's rows of the first tensor
  // At most kFusedInFlight rows of a thread are in flight: with every row of the grid requested
  // at once the memory system serves some waves far later than the others, and every block
  // waits for the slowest part of its slab.
  v4u v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    v[k] = __builtin_nontemporal_load(row_of(a.x, k));
    if (k >= kFusedInFlight) asm volatile("" : "+v"(v[k - kFusedInFlight])::"memory");
  }
  // range of the thread's 8 channels over its rows, on the raw bits (written out here: a helper
  // or lambda that takes the row array by reference leaves it in scratch memory)
  float lo[8], hi[8];
  uint32_t hb[4] = {0u, 0u, 0u, 0u}, lb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hb[j] = pk_max_i16(hb[j], w[j]);
      lb[j] = pk_max_u16(lb[j], w[j]);
    }
  }
  range_from_bits(hb, lb, lo, hi);
  // keep only the packed rows live across the exchange (the codes decode them again)
#pragma unroll
  for (int k = 0; k < R; ++k) asm volatile("" : "+v"(v[k]));
  fused_slab_params(sh, a, lo, hi, tokens, channels, slab, part, epoch, spin_ticks);

  float s8[8], r8[8], z8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s8[i] = sh.prm[0][lc * 8 + i];
    r8[i] = sh.prm[1][lc * 8 + i];
    z8[i] = sh.prm[2][lc * 8 + i];
  }
  uint8_t* qp = a.q + (size_t)(t0 + rr) * channels + c0;
  if constexpr (!kPair) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k < nk) __builtin_nontemporal_store(quant_row8(v[k], s8, r8, z8), reinterpret_cast<v2u*>(qp));
      qp += pass;
    }
  } else {
    // ---- codes of the first tensor, each row's register refilled with the second's row
    // The second tensor's rows come from a moving pointer (rows past the tensor's end read its
    // last row, as row_of does), kept opaque so that the compiler does not precompute every
    // row's address ahead of the loop: those addresses would not fit beside the rows.
    const uint16_t* xb = b.x + (size_t)(t0 + rr) * channels + c0;
    const uint16_t* const xlast = b.x + (size_t)(tokens - 1) * channels + c0;
    const int rem = tokens - 1 - t0 - rr;
    const int klast = rem < 0 ? -1 : rem / kFusedRowsPerPass;  // last row k inside the tensor
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k < nk) __builtin_nontemporal_store(quant_row8(v[k], s8, r8, z8), reinterpret_cast<v2u*>(qp));
      qp += pass;
      v[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(k <= klast ? xb : xlast));
      xb += pass;
      asm volatile("" : "+v"(xb));
      if (k >= kPairInFlight) asm volatile("" : "+v"(v[k - kPairInFlight])::"memory");
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) hb[j] = lb[j] = 0u;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hb[j] = pk_max_i16(hb[j], w[j]);
        lb[j] = pk_max_u16(lb[j], w[j]);
      }
    }
    range_from_bits(hb, lb, lo, hi);
#pragma unroll
    for (int k = 0; k < R; ++k) asm volatile("" : "+v"(v[k]));
    // the first tensor's parameters were read into registers before any thread could reach
    // the barriers of this second exchange, so sh.prm may be rewritten
    fused_slab_params(sh, b, lo, hi, tokens, channels, slab, part, epoch, spin_ticks);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s8[i] = sh.prm[0][lc * 8 + i];
      r8[i] = sh.prm[1][lc * 8 + i];
      z8[i] = sh.prm[2][lc * 8 + i];
    }
    qp = b.q + (size_t)(t0 + rr) * channels + c0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k < nk) __builtin_nontemporal_store(quant_row8(v[k], s8, r8, z8), reinterpret_cast<v2u*>(qp));
      qp += pass;
    }
  }
}

// ---------------------------------------------------------------- host side
static int fused_rows(int tokens, int channels) {
  if (channels % kFusedCh != 0 || tokens <= 0) return 0;
  const long long per = ((long long)tokens + kFusedParts - 1) / kFusedParts;
  const long long rows = (per + kFusedRowsPerPass - 1) / kFusedRowsPerPass;
  return rows <= kFusedMaxRows ? (int)rows : 0;
}

// One size serves both calls: the paired call's two fused regions, or the three-pass
// schedule's partials (which the paired call's fallback uses for one tensor after the other).
size_t kv_workspace_bytes(int tokens, int channels) {
  if (tokens <= 0 || channels <= 0) return 0;
  const size_t three_pass = (size_t)2 * kv_range_chunks(tokens) * channels * sizeof(float);
  const size_t fused = 2 * fused_region_bytes(channels);
  return three_pass > fused ? three_pass : fused;
}

// Epoch of a fused call: strictly increasing per process and never 0, started at a
// time-dependent value, so a word left in a workspace by an earlier call of this process never
// carries the running call's epoch (what the memory held before, from elsewhere, matches with
// chance 2^-32 per word).
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

template <bool kPair>
static const void* fused_fn(int n) {
  switch (n) {
    case 1: return reinterpret_cast<const void*>(&kv_quant_fused_kernel<8, kPair>);
    case 2: return reinterpret_cast<const void*>(&kv_quant_fused_kernel<16, kPair>);
    case 3: return reinterpret_cast<const void*>(&kv_quant_fused_kernel<24, kPair>);
    case 4: return reinterpret_cast<const void*>(&kv_quant_fused_kernel<32, kPair>);
    case 5: return reinterpret_cast<const void*>(&kv_quant_fused_kernel<40, kPair>);
    default: return nullptr;
  }
}

// Blocks of kv_quant_fused_kernel<8 n, pair> that the current device holds at once (0 if
// unknown).  The exchange waits for every part of a slab, so the fused pass is launched only
// when the whole grid is resident together; the bounded wait stays as the guard for anything
// else sharing the device.
static int fused_resident_blocks(int n, bool pair) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][2][6];  // value + 1; 0 = not yet queried
  int dev = 0;
  if (n < 1 || n > 5 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int c = cache[dev][pair][n].load(std::memory_order_relaxed);
  if (c) return c - 1;
  int per_cu = 0, cus = 0;
  const void* fn = pair ? fused_fn<true>(n) : fused_fn<false>(n);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kFusedThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error behind; use the three-pass path
    return 0;
  }
  const int blocks = per_cu * cus;
  cache[dev][pair][n].store(blocks + 1, std::memory_order_relaxed);
  return blocks;
}

// Rows per thread of the fused launch for this shape, or 0 when the three-pass schedule runs.
static int fused_choice(int tokens, int channels, bool pair) {
  const int rows = fused_rows(tokens, channels);
  if (rows == 0) return 0;
  const int n = (rows + 7) / 8;
  return (channels / kFusedCh) * kFusedParts <= fused_resident_blocks(n, pair) ? n : 0;
}

template <bool kPair>
static hipError_t launch_fused(int n, const KvFusedTensor& a, const KvFusedTensor& b, int tokens,
                               int channels, hipStream_t stream) {
  const dim3 grid((channels / kFusedCh) * kFusedParts), block(kFusedThreads);
  const uint32_t epoch = next_epoch();
  const long long ticks = spin_ticks();
  switch (n) {
#define SVDQ_KV_FUSED(n)                                                                        \
  case n:                                                                                       \
    hipLaunchKernelGGL((kv_quant_fused_kernel<8 * n, kPair>), grid, block, 0, stream, a, b,     \
                       tokens, channels, epoch, ticks);                                         \
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

static KvFusedTensor fused_tensor(const uint16_t* x, uint8_t* q, float* scale, uint8_t* zero,
                                  void* region) {
  return KvFusedTensor{x, q, scale, zero, reinterpret_cast<uint64_t*>(region)};
}

static hipError_t launch_three_pass(const uint16_t* x, int tokens, int channels, uint8_t* q,
                                    float* scale, uint8_t* zero, void* workspace,
                                    hipStream_t stream) {
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

hipError_t launch_kv_quant(const uint16_t* x, int tokens, int channels, uint8_t* q,
                           float* scale, uint8_t* zero, void* workspace, hipStream_t stream) {
  if (const int n = fused_choice(tokens, channels, false)) {
    const KvFusedTensor a = fused_tensor(x, q, scale, zero, workspace);
    return launch_fused<false>(n, a, a, tokens, channels, stream);
  }
  return launch_three_pass(x, tokens, channels, q, scale, zero, workspace, stream);
}

hipError_t launch_kv_quant_pair(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                                uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv,
                                uint8_t* zv, void* workspace, hipStream_t stream) {
  if (const int n = fused_choice(tokens, channels, true)) {
    const KvFusedTensor a = fused_tensor(k, qk, sk, zk, workspace);
    const KvFusedTensor b = fused_tensor(
        v, qv, sv, zv, reinterpret_cast<uint8_t*>(workspace) + fused_region_bytes(channels));
    return launch_fused<true>(n, a, b, tokens, channels, stream);
  }
  // one tensor after the other on the stream, sharing the workspace
  const hipError_t e = launch_kv_quant(k, tokens, channels, qk, sk, zk, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_kv_quant(v, tokens, channels, qv, sv, zv, workspace, stream);
}

// ---------------------------------------------------------------- allocation-free variant
// Device scratch of kv_int8_quant_pair_noalloc: a file-scope array that every device the library
// runs on holds until the process ends.  Host code never passes the array's name to a kernel or
// a copy (on the host it is only a stand-in): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.  Nothing in
// it needs to start at zero (the single pass accepts only words tagged with the running call's
// epoch; the three-pass schedule writes every partial before reading it); calls that overlap in
// time on one device share it and race.
static __device__ __align__(256) unsigned char scratch[kKvStaticScratchBytes];

static hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_kv_quant_pair_noalloc(const uint16_t* k, const uint16_t* v, int tokens,
                                        int channels, uint8_t* qk, float* sk, uint8_t* zk,
                                        uint8_t* qv, float* sv, uint8_t* zv, hipStream_t stream) {
  if (kv_workspace_bytes(tokens, channels) > kKvStaticScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_kv_quant_pair(k, v, tokens, channels, qk, sk, zk, qv, sv, zv, ws, stream);
}

hipError_t launch_kv_dequant(const uint8_t* q, const float* scale, const uint8_t* zero,
                             int tokens, int channels, uint16_t* x_out, hipStream_t stream) {
  const dim3 grid(kv_slabs(channels), (tokens + kDeqTokPerBlock - 1) / kDeqTokPerBlock);
  hipLaunchKernelGGL(kv_dequant_kernel, grid, dim3(256), 0, stream, q, scale, zero, tokens,
                     channels, x_out);
  return hipGetLastError();
}

}  // namespace svdq
