// Device helpers shared by the gfx950 kernels: exact quantizer rounding, fp16/bf16 conversion,
// nibble unpacking onto int8 MFMA operands and the MFMA vector types.
//
// Every kernel file is compiled with -ffp-contract=off: each rounding step written here is the
// rounding the contract asks for, and fused multiply-adds appear only where a kernel calls
// __builtin_fmaf itself (the GEMM's dequantization, which is tolerance-checked).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;  // quantization group along K

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default rounding mode).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> one dword of two bf16 (lo in bits 0..15), each rounded to nearest even.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return (uint32_t)float_to_bf16_bits(lo) | ((uint32_t)float_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- exact quantizer rounding
// rne(fl32(x / s)) for s != 0, given rcp = fl32(1 / s).  The product t = fl32(x * rcp) lies
// within |x/s| * 2^-22.4 of fl32(x / s); the two can only round to different integers when t
// is that close to a half-integer, so within a (much wider) window of 2^-20 * max(1, |t|)
// around a half-integer the quotient is recomputed with the IEEE division.
__device__ __forceinline__ float rne_quotient(float x, float s, float rcp) {
  float t = x * rcp;
  float r = __builtin_rintf(t);
  float d = __builtin_fabsf(t - r);
  if (__builtin_fabsf(d - 0.5f) <= 0x1p-20f * __builtin_fmaxf(1.0f, __builtin_fabsf(t))) {
    r = __builtin_rintf(x / s);
  }
  return r;
}

// Symmetric INT4 scale of a group from its max magnitude: fp16(fl32(amax / 7)).
__device__ __forceinline__ uint16_t int4_scale_bits(float amax) {
  return float_to_half_bits(amax / 7.0f);
}

// Code in [-8, 7] of one value given the group's fp16 scale (as fp32, nonzero) and 1/scale.
__device__ __forceinline__ int int4_code(float x, float s, float rcp) {
  float r = rne_quotient(x, s, rcp);
  r = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  return (int)r;
}

// ---------------------------------------------------------------- nibble unpack
// Sixteen packed two's-complement nibbles (two dwords; in each, k0 in bits 0..3, ..., k7 in
// bits 28..31) become four dwords of int8 lanes holding 16 * code: per packed dword, one with
// k0,k2,k4,k6 and one with k1,k3,k5,k7.  Placing a
// nibble in the high half of a byte multiplies it by 16 exactly, so the int8 dot product of
// two unpacked operands is 256 times the code dot product.  The k order inside the dwords is a
// permutation of the packed order; it is the same for both GEMM operands, and a dot product is
// invariant under a permutation applied to both.
__device__ __forceinline__ v4i unpack16_x16(v2u v) {
  return v4i{(int)((v.x << 4) & 0xF0F0F0F0u), (int)(v.x & 0xF0F0F0F0u),
             (int)((v.y << 4) & 0xF0F0F0F0u), (int)(v.y & 0xF0F0F0F0u)};
}

}  // namespace svdq
