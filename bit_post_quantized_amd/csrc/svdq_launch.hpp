// Host-side launchers of the gfx950 kernels (one per kernel file).  Arguments are validated by
// the C ABI layer before any of these is called; each returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

// e3m2 != 0: write the codes into the tiled BF6 container instead of nibbles [rows, K/2]
hipError_t launch_pack_weights(const float* R, int K, int N, uint8_t* wq, uint16_t* w_scales,
                               int e3m2, hipStream_t stream);

// L1 [K, r] -> L1p [r, K] (the activation pass's layout of the low-rank factor)
hipError_t launch_pack_lowrank(const uint16_t* L1, int K, int r, uint16_t* L1p,
                               hipStream_t stream);

// L2 [r, N] -> L2p [N, r] (the GEMM epilogue's layout of the up-projection factor)
hipError_t launch_pack_lowrank_up(const uint16_t* L2, int r, int N, uint16_t* L2p,
                                  hipStream_t stream);

// code containers of the activation pass: INT4 as nibbles [M, K/2], INT4 as the tiled BF6
// container, or the 8-bit codes of the W4A8 variant [M, K] (int8)
constexpr int kCodesNibbles = 0, kCodesBf6 = 1, kCodesInt8 = 2;

hipError_t launch_quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                               int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                               int codes, hipStream_t stream);

hipError_t launch_w4a4_gemm(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                            const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                            const uint16_t* bias, int M, int N, int K, int r, void* Y,
                            int out_fp32, int32_t* partials, hipStream_t stream);

// W4A8: int8 activation codes [M, K] times the INT4 weight nibbles, on the INT8 matrix units
hipError_t launch_w4a8_gemm(const uint8_t* xq8, const uint16_t* x_scales, const float* T,
                            const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                            const uint16_t* bias, int M, int N, int K, int r, void* Y,
                            int out_fp32, int32_t* partials, hipStream_t stream);

hipError_t launch_w4a4_gemm_e3m2(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                                 const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                                 const uint16_t* bias, int M, int N, int K, int r, void* Y,
                                 int out_fp32, int32_t* partials, hipStream_t stream);

size_t kv_workspace_bytes(int tokens, int channels);

hipError_t launch_kv_quant(const uint16_t* x, int tokens, int channels, uint8_t* q,
                           float* scale, uint8_t* zero, void* workspace, hipStream_t stream);

hipError_t launch_kv_quant_pair(const uint16_t* k, const uint16_t* v, int tokens, int channels,
                                uint8_t* qk, float* sk, uint8_t* zk, uint8_t* qv, float* sv,
                                uint8_t* zv, void* workspace, hipStream_t stream);

// scratch that kv_int8_quant_pair_noalloc holds per device (16 MiB)
constexpr size_t kKvStaticScratchBytes = (size_t)16 << 20;
hipError_t launch_kv_quant_pair_noalloc(const uint16_t* k, const uint16_t* v, int tokens,
                                        int channels, uint8_t* qk, float* sk, uint8_t* zk,
                                        uint8_t* qv, float* sv, uint8_t* zv, hipStream_t stream);

hipError_t launch_kv_dequant(const uint8_t* q, const float* scale, const uint8_t* zero,
                             int tokens, int channels, uint16_t* x_out, hipStream_t stream);

// decode attention over the INT8 cache (codes, per-channel scale / zero of K and V)
size_t kv_attn_workspace_bytes(int nq, int tokens, int heads, int dim);

hipError_t launch_kv_attention(const uint16_t* q, const uint8_t* kq, const float* ks,
                               const uint8_t* kz, const uint8_t* vq, const float* vs,
                               const uint8_t* vz, int nq, int tokens, int heads, int dim,
                               float sm_scale, uint16_t* out, void* workspace,
                               hipStream_t stream);

}  // namespace svdq
