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
// fl32(x / s), correctly rounded, without a division per element: with rcp = fl32(1 / s),
// q0 = fl32(x * rcp) is within one ulp of x / s, the residual x - q0 * s is exact in one FMA,
// and one more FMA rounds q0 + residual * rcp to the correctly rounded quotient (Markstein's
// correction step for division with an accurate reciprocal; valid away from underflow, which
// the codes never reach: a quotient below 2^-100 rounds to code 0 either way).
__device__ __forceinline__ float div_rn(float x, float s, float rcp) {
  const float q0 = x * rcp;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(r, rcp, q0);
}

// rne(fl32(x / s)) for s != 0, given rcp = fl32(1 / s).
__device__ __forceinline__ float rne_quotient(float x, float s, float rcp) {
  return __builtin_rintf(div_rn(x, s, rcp));
}

// Symmetric INT4 scale of a group from its max magnitude: fp16(fl32(amax / 7)).
__device__ __forceinline__ uint16_t int4_scale_bits(float amax) {
  return float_to_half_bits(amax / 7.0f);
}

// Codes of a whole 64-group, packed eight per dword (even k in the low nibble):
// q = clamp(rne(fl32(x / s)), -8, 7), biased by 8, converted to bytes (v_cvt_pk_u8_f32),
// merged pairwise into nibbles and un-biased by flipping bit 3 of every nibble.
__device__ __forceinline__ void quantize_group_int4(const float* x, float s, uint32_t* packed) {
  if (s == 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) packed[j] = 0u;
    return;
  }
  const float rcp = 1.0f / s;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t ev = 0u, od = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = rne_quotient(x[8 * j + 2 * e], s, rcp);
      const float b = rne_quotient(x[8 * j + 2 * e + 1], s, rcp);
      ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(a + 8.0f, 0.0f, 15.0f), e, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(b + 8.0f, 0.0f, 15.0f), e, od);
    }
    packed[j] = ((od << 4) | ev) ^ 0x88888888u;
  }
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
