// Peak microbenchmarks for the benchmark's "% of measured peak" figures: how fast this device
// issues the matrix instructions the linear layer uses, and how fast it streams HBM.
//
//  * peaks_mfma: every wave issues `iters` rounds of 8 independent 32x32 MFMAs of one kind
//    (FP6 E3M2 32x32x64 with unit scales, INT8 32x32x32, bf16 32x32x16) into 8 accumulators,
//    then folds them into one float per wave (so no MFMA is dead code).  The operands are
//    lane-dependent values fixed for the whole loop: only the matrix pipe's issue rate is
//    measured, with no memory traffic.
//  * peaks_copy: a device-to-device copy with 16-byte non-temporal loads and stores (grid-stride
//    over a given grid, or one workgroup per contiguous 16 KiB or 64 KiB run), the plain HBM
//    stream (read + write bytes).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "svdq_peaks.h"

namespace {

typedef int pk_v4i __attribute__((ext_vector_type(4)));
typedef int pk_v8i __attribute__((ext_vector_type(8)));
typedef int pk_v16i __attribute__((ext_vector_type(16)));
typedef float pk_v16f __attribute__((ext_vector_type(16)));
typedef __bf16 pk_v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int pk_v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 8;

__device__ __forceinline__ float fold16(const pk_v16f& a) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += a[i];
  return s;
}

template <int Kind>
__global__ __launch_bounds__(kThreads) void mfma_loop(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  float sum = 0.0f;
  if constexpr (Kind == PEAKS_FP6) {
    pk_v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x01041041 * ((lane + i) & 7);  // small E3M2 codes in every 6-bit slot
      b[i] = 0x00820820 * ((lane + 3 * i) & 7);
    }
    pk_v16f acc[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 3, 3, 0, 127, 0, 127);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) sum += fold16(acc[c]);
  } else if constexpr (Kind == PEAKS_INT8) {
    pk_v4i a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 3);
      b[i] = 0x01010101 * ((lane + 2 * i) & 3);
    }
    pk_v16i acc[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += (float)acc[c][i];
  } else {
    pk_v8bf a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.25f * ((lane + i) & 3));
      b[i] = (__bf16)(0.5f * ((lane + 2 * i) & 3));
    }
    pk_v16f acc[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) sum += fold16(acc[c]);
  }
  if (lane == 0) out[(size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = sum;
}

__global__ __launch_bounds__(kThreads) void copy_stream(const pk_v4u* __restrict__ src,
                                                        pk_v4u* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  // four 16-byte loads in flight per thread, then their stores
  for (; i + 3 * stride < n; i += 4 * stride) {
    pk_v4u v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], dst + i + k * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// one block copies a contiguous run of kThreads * RUN 16-byte vectors, every load in flight
// before its stores
template <int RUN>
__global__ __launch_bounds__(kThreads) void copy_runs(const pk_v4u* __restrict__ src,
                                                      pk_v4u* __restrict__ dst, size_t n) {
  const size_t base = (size_t)blockIdx.x * kThreads * RUN + threadIdx.x;
  pk_v4u v[RUN];
#pragma unroll
  for (int k = 0; k < RUN; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < RUN; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n) __builtin_nontemporal_store(v[k], dst + i);
  }
}

template <int RUN>
static hipError_t launch_runs(const pk_v4u* s, pk_v4u* d, size_t n, hipStream_t stream) {
  const size_t runs = (n + (size_t)kThreads * RUN - 1) / ((size_t)kThreads * RUN);
  if (runs > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_runs<RUN>, dim3((unsigned)runs), dim3(kThreads), 0, stream, s, d, n);
  return hipGetLastError();
}

double flops_per_mfma(int kind) {
  switch (kind) {
    case PEAKS_FP6: return 2.0 * 32 * 32 * 64;
    case PEAKS_INT8: return 2.0 * 32 * 32 * 32;
    case PEAKS_BF16: return 2.0 * 32 * 32 * 16;
    default: return 0.0;
  }
}

}  // namespace

extern "C" {

double peaks_mfma_flops(int kind, int blocks, int iters) {
  if (blocks <= 0 || iters <= 0) return 0.0;
  return flops_per_mfma(kind) * kChains * (double)iters * (double)blocks * (kThreads / 64);
}

size_t peaks_mfma_out_floats(int blocks) {
  return blocks > 0 ? (size_t)blocks * (kThreads / 64) : 0;
}

int peaks_mfma(int kind, int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || blocks > 1 << 20 || iters <= 0 || !out) return 1;
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case PEAKS_FP6:
      hipLaunchKernelGGL(mfma_loop<PEAKS_FP6>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
      break;
    case PEAKS_INT8:
      hipLaunchKernelGGL(mfma_loop<PEAKS_INT8>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
      break;
    case PEAKS_BF16:
      hipLaunchKernelGGL(mfma_loop<PEAKS_BF16>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
      break;
    default:
      return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int peaks_copy(const void* src, void* dst, size_t bytes, int mode, int blocks, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0) return 1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 3;
  const size_t n = bytes / 16;
  const auto* s = reinterpret_cast<const pk_v4u*>(src);
  auto* d = reinterpret_cast<pk_v4u*>(dst);
  hipError_t e;
  switch (mode) {
    case PEAKS_COPY_STRIDE:
      if (blocks <= 0 || blocks > 1 << 20) return 1;
      hipLaunchKernelGGL(copy_stream, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, s, d,
                         n);
      e = hipGetLastError();
      break;
    case PEAKS_COPY_RUNS_16K:
      e = launch_runs<4>(s, d, n, (hipStream_t)stream);
      break;
    case PEAKS_COPY_RUNS_64K:
      e = launch_runs<16>(s, d, n, (hipStream_t)stream);
      break;
    default:
      return 1;
  }
  return e == hipSuccess ? 0 : 4;
}

}  // extern "C"
