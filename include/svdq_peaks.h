/*
 * svdq_peaks.h — microbenchmarks of the device's own peaks (libsvdq_peaks.so), the denominators
 * of the benchmark's "% of measured peak" figures.  They compute nothing of the method: the
 * matrix loops measure how fast a device issues the instruction kinds the linear layer runs on,
 * the copy how fast it streams HBM.  All pointers are device pointers; launches are
 * asynchronous on `stream` (a hipStream_t, NULL for the default stream).
 *
 * Status: 0 ok, 1 invalid argument, 3 misaligned pointer, 4 the HIP runtime refused the launch.
 */
#ifndef SVDQ_PEAKS_H
#define SVDQ_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum peaks_kind {
  PEAKS_FP6 = 0,  /* v_mfma_scale_f32_32x32x64_f8f6f4, E3M2 x E3M2, unit scales */
  PEAKS_INT8 = 1, /* v_mfma_i32_32x32x32_i8 */
  PEAKS_BF16 = 2  /* v_mfma_f32_32x32x16_bf16 */
};

/*
 * peaks_mfma — `blocks` workgroups of 256 threads; every wave issues `iters` rounds of 8
 * independent MFMAs of `kind` and writes one float to out[block * 4 + wave].
 *   out  fp32 [peaks_mfma_out_floats(blocks)], caller-owned.
 *   1 <= blocks <= 2^20, iters >= 1.
 * peaks_mfma_flops gives the launch's arithmetic (2 m n k per MFMA; integer ops for INT8).
 */
int peaks_mfma(int kind, int blocks, int iters, float* out, void* stream);
double peaks_mfma_flops(int kind, int blocks, int iters);
size_t peaks_mfma_out_floats(int blocks);

/*
 * peaks_copy — dst[0, bytes) = src[0, bytes) with 16-byte non-temporal loads and stores over
 * workgroups of 256 threads, by launch shape `mode`:
 *   PEAKS_COPY_STRIDE    `blocks` workgroups striding over the range, 4 loads in flight per
 *                        thread (1 <= blocks <= 2^20);
 *   PEAKS_COPY_RUNS_16K  one workgroup per contiguous 16 KiB run (4 loads per thread);
 *   PEAKS_COPY_RUNS_64K  one workgroup per contiguous 64 KiB run (16 loads per thread).
 * bytes % 16 == 0, both pointers 16-byte aligned, the ranges disjoint.
 */
enum peaks_copy_mode { PEAKS_COPY_STRIDE = 0, PEAKS_COPY_RUNS_16K = 1, PEAKS_COPY_RUNS_64K = 2 };
int peaks_copy(const void* src, void* dst, size_t bytes, int mode, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_PEAKS_H */
