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
typedef unsigned int v3u __attribute__((ext_vector_type(3)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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

// fl32(1 / s) for s an fp16 value held in fp32 (s != 0): the hardware reciprocal, which is within
// one ulp, refined by one correction step y + y (1 - s y) in two FMAs.  For every fp16
// significand and every start within two ulps of 1 / s this is the correctly rounded
// reciprocal (an exact-rational enumeration of all 1024 significands); 1 / s of an fp16 is a
// normal fp32, so the exponent only scales.
__device__ __forceinline__ float rcp_rn_half(float s) {
  const float y = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y, 1.0f);
  return __builtin_fmaf(e, y, y);
}

// fp16(fl32(amax / d)) with the quotient by the correction step above and the correctly rounded
// constant fl32(1 / d) (a quotient in fp32's subnormal range rounds to an fp16 zero either way).
// The fp32 quotient is kept opaque before the conversion: left to itself the compiler fuses the
// last FMA with the conversion (v_fma_mixlo_f16), which rounds once, straight to fp16, and
// differs from the two roundings the scale is defined by.
template <int D>
__device__ __forceinline__ uint16_t scale_bits_div(float amax) {
  constexpr float kRcp = 1.0f / (float)D;
  float q = div_rn(amax, (float)D, kRcp);
  asm volatile("" : "+v"(q));
  return float_to_half_bits(q);
}

// Symmetric INT4 scale of a group from its max magnitude: fp16(fl32(amax / 7)).
__device__ __forceinline__ uint16_t int4_scale_bits(float amax) { return scale_bits_div<7>(amax); }

// The 8-bit variant's scale fp16(fl32(amax / 127)).
__device__ __forceinline__ uint16_t int8_scale_bits(float amax) { return scale_bits_div<127>(amax); }

// Eight codes (floats holding integers in [-8, 7]) -> one dword of nibbles, code i in bits
// 4i .. 4i+3, two's complement: bias by 8, convert to bytes, merge even / odd, un-bias.
__device__ __forceinline__ uint32_t pack8_nibbles(const float* c) {
  uint32_t ev = 0u, od = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ev = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * e] + 8.0f, e, ev);
    od = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * e + 1] + 8.0f, e, od);
  }
  return ((od << 4) | ev) ^ 0x88888888u;
}

// ---------------------------------------------------------------- BF6 (E3M2) container
// BF6 as defined by the OCP Microscaling format: sign bit 5, exponent bits 4..2 with bias 3,
// mantissa bits 1..0.  An fp32 holding an integer code in [-8, 8] has at most two significant
// mantissa bits after the leading one, so its E3M2 pattern is read straight out of the fp32
// pattern: bits 30..21 hold (exponent + 127) << 2 | mantissa[22:21], and 127 - 3 = 124,
// 124 << 2 = 496.  Both zeros map to +0.
__device__ __forceinline__ uint32_t e3m2_of_code(float c) {
  const uint32_t b = __float_as_uint(c);
  const uint32_t p = (((b >> 21) & 0x3FFu) - 496u) | ((b >> 26) & 0x20u);
  return (b << 1) == 0u ? 0u : p;
}

// Tiled BF6 container of a [R, K] code matrix: ceil(R / 32) row blocks; block b holds, group by
// group, 64 slots of 24 bytes; slot s carries the 32 codes of row 32 b + s % 32 at
// k = 64 g + 32 (s / 32) + i as one 192-bit stream -- the lane order of the 32 x 32 x 64 FP6
// MFMA operand, so a GEMM stage is a plain copy of whole blocks.
constexpr int kE3m2Rows = 32;
constexpr int kE3m2Block = 64 * 24;  // one row block x one group

// Sixteen codes -> three dwords of the packed little-endian stream (code i at bits 6i..6i+5).
__device__ __forceinline__ v3u pack16_e3m2(const float* c) {
  uint32_t p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = e3m2_of_code(c[i]);
  const uint32_t w0 = p[0] | (p[1] << 6) | (p[2] << 12) | (p[3] << 18) | (p[4] << 24) | (p[5] << 30);
  const uint32_t w1 = (p[5] >> 2) | (p[6] << 4) | (p[7] << 10) | (p[8] << 16) | (p[9] << 22) | (p[10] << 28);
  const uint32_t w2 = (p[10] >> 4) | (p[11] << 2) | (p[12] << 8) | (p[13] << 14) | (p[14] << 20) | (p[15] << 26);
  return v3u{w0, w1, w2};
}

// ---------------------------------------------------------------- codes as biased bytes
// The activation pass turns each code c in [-8, 7] into the byte c + 8 (v_cvt_pk_u8_f32 of an
// exact small integer), then derives either container from four bytes at a time.

// Four fp32 holding integers in [0, 15] -> one dword of bytes, value i in byte i.
__device__ __forceinline__ uint32_t bytes4(const float* v) {
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) w = __builtin_amdgcn_cvt_pk_u8_f32(v[i], i, w);
  return w;
}

// Eight biased codes (two dwords of bytes) -> one dword of nibbles, code i in bits 4i .. 4i+3,
// two's complement: OR each dword with itself shifted by 4 so bytes 0 and 2 hold two codes
// each, gather those bytes with v_perm_b32, and flip bit 3 of every nibble (c + 8 xor 8 is the
// 4-bit two's complement of c).
__device__ __forceinline__ uint32_t nibbles8_biased(uint32_t lo, uint32_t hi) {
  const uint32_t x = lo | (lo >> 4), y = hi | (hi >> 4);
  return __builtin_amdgcn_perm(y, x, 0x06040200u) ^ 0x88888888u;
}

// Four biased codes (bytes c + 8) -> four BF6 (E3M2) patterns, one per byte, by table lookup.
// v_perm_b32 returns, per selector byte 0..7, that byte of the 8-byte pool {src0, src1} (src1
// holds bytes 0..3); selector 0x0C gives 0x00 and 0x0D gives 0xFF.  One table holds the
// patterns of c = -8..-1, one those of c = 0..7 (0x00 0C 10 12 14 15 16 17: 0, 1, 2, 3, 4, 5,
// 6, 7; the negative ones add the sign bit 0x20, -8 is 0x38), and bit 3 of each byte picks
// between them through a byte mask made by a third v_perm_b32.
__device__ __forceinline__ uint32_t bf6_of_biased4(uint32_t b) {
  const uint32_t sel = b & 0x07070707u;
  const uint32_t neg = __builtin_amdgcn_perm(0x2C303234u, 0x35363738u, sel);
  const uint32_t pos = __builtin_amdgcn_perm(0x17161514u, 0x12100C00u, sel);
  const uint32_t msk = __builtin_amdgcn_perm(0u, 0u, ((b >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  return (pos & msk) | (neg & ~msk);
}

// Four 6-bit patterns in bytes -> one 24-bit run, pattern i at bits 6i.
__device__ __forceinline__ uint32_t pack4_bf6(uint32_t p) {
  const uint32_t t = (p & 0x003F003Fu) | ((p >> 2) & 0x0FC00FC0u);  // p0 | p1<<6 | p2<<16 | p3<<22
  return (t & 0xFFFu) | ((t >> 4) & 0xFFF000u);
}

// Sixteen biased codes (four dwords of bytes) -> three dwords of the BF6 stream (code i at bits
// 6i .. 6i+5), the same stream pack16_e3m2 writes.
__device__ __forceinline__ v3u pack16_bf6_biased(const uint32_t* b) {
  const uint32_t c0 = pack4_bf6(bf6_of_biased4(b[0])), c1 = pack4_bf6(bf6_of_biased4(b[1]));
  const uint32_t c2 = pack4_bf6(bf6_of_biased4(b[2])), c3 = pack4_bf6(bf6_of_biased4(b[3]));
  return v3u{c0 | (c1 << 24), (c1 >> 8) | (c2 << 16), (c2 >> 16) | (c3 << 8)};
}

// Eight fp32 -> eight bf16 (round to nearest even, v_cvt_pk_bf16_f32) as an MFMA operand.
__device__ __forceinline__ v8bf to_bf16x8(const float* x) {
  v4u a;
  a.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{x[0], x[1]}), v2bf));
  a.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{x[2], x[3]}), v2bf));
  a.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{x[4], x[5]}), v2bf));
  a.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{x[6], x[7]}), v2bf));
  return __builtin_bit_cast(v8bf, a);
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

// XCD-aware tile order for a GEMM grid of (column tiles, row tiles).  Workgroups go to the 8
// XCDs round-robin by linear id, and each XCD has its own L2: linear id L runs on XCD L % 8 as
// that XCD's (L / 8)-th workgroup, so it takes logical tile (L % 8) T / 8 + L / 8 (a bijection
// on the first 8 floor(T / 8) ids; the rest keep their id) and each XCD walks a contiguous run
// of logical tiles.  Logical tiles go in bands of `band` row tiles, row tile fastest: the
// workgroups an XCD runs at once share `band` activation panels and a few weight panels, which
// stay in its L2 while it sweeps the columns.  Returns (row tile, column tile).  The int
// arithmetic holds: the GEMMs' 128 x 128 tiles and M N <= 2^40 keep T below 2^27.
__device__ __forceinline__ void xcd_tile_order(int band, int& mt, int& nt) {
  const int nx = gridDim.x, ny = gridDim.y, T = nx * ny, T8 = T / 8 * 8;
  int L = blockIdx.y * nx + blockIdx.x;
  if (L < T8) L = (L % 8) * (T / 8) + L / 8;
  const int b = L / (band * nx), first = b * band;
  const int rows = min(ny - first, band), within = L - b * band * nx;
  mt = first + within % rows;
  nt = within / rows;
}

}  // namespace svdq
