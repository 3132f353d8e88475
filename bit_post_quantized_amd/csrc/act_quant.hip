// Fused activation pass: smoothing, dynamic low-bit quantization and the low-rank
// down-projection.
//
// SVDQ "technical principles": smoothing moves activation outliers into the weights, and a
// 16-bit low-rank branch runs beside the 4-bit one.  FLUX4 3.1: activations are quantized at
// run time.  W4A8 3.1: symmetric scale max|v| / (2^(b-1) - 1), round, clamp, one scale per
// token and 64-group; b = 4 (INT4 codes) or b = 8 (the W4A8 variant's activations, W4A8 1).
// SVDQ / DCMP: the branch is fused so the activations are read from HBM once.
//
// Work decomposition.  A workgroup owns 16 tokens (rows) and all of K, or half of K (long K),
// or, with long K and more row blocks than CUs, an equal share of the (row block, group) units
// that may span three row blocks; its waves take the 64-groups round-robin.  In a group, lane l holds row l / 4 and the 16 consecutive k
// [16 q, 16 q + 16) of quarter q = l % 4: two 16-byte loads, and the four lanes of a quad read
// one row's 128 contiguous bytes.  (The vector memory unit resolves a 16-byte load four lanes
// at a time; with the four lanes of a quad on four different rows, the same loads took twice
// as long.)  The loads of kActBatch groups are issued before any of them is used; inv_lambda
// sits in LDS.  The group max is folded over the quad with two DPP lane swaps; every lane then
// codes its 16 values (exact quotient, no division per element) as biased bytes c + 2^(b-1)
// and writes them in one of three containers: 8 bytes of
// nibbles, 12 bytes of BF6 (E3M2) patterns into the tiled container (its row block, group,
// slot row % 32 + 32 (q / 2), byte 12 (q % 2)), or 16 bytes of int8.  The quarter-0 lanes write
// the 16 rows' scales.  For the tiled container the grid also covers the rows up to the next
// multiple of 32, whose codes it writes as zeros.
// Low-rank branch: the same registers rounded to bf16, and L1 (stored K-contiguous, loaded
// with the same quad-per-row map: rank row 16 t + l / 4, quarter l % 4), are moved by a fixed
// lane permutation (ds_bpermute: lane l takes lane 4 (l % 16) + l / 16) into the operand
// layout of v_mfma_f32_16x16x32_bf16, row or column l % 16 and k-slots 8 (l / 16) + i; two
// MFMAs per group take k = 16 q + i and 16 q + 8 + i, so they sum exactly the group's 64 k.
// Per-wave partial T tiles are summed in LDS in wave order (deterministic) and written once,
// or, where two workgroups share a row block, added atomically onto a zeroed T (two additions:
// deterministic, but at long K the rounding of T then depends on where the shares fall).
#include <atomic>

#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v6u __attribute__((ext_vector_type(6)));

constexpr int kActRows = 16;    // tokens per workgroup
// Waves per workgroup and groups per wave whose code loads are in flight together, by the
// rank's 16-wide tiles NTR.  Eight waves share a workgroup's groups.  Up to rank 32 they stay
// within 128 VGPRs, so two workgroups share a CU and a 4608-row pass (288 workgroups) is
// resident at once: 16 waves per workgroup (one workgroup per CU, 256 in a first round and 32
// in a second) took 23.2 against 20.9 us inside the bench step.  A wave keeps a batch of
// groups in flight and refills each slot with the next batch's group once it has been read:
// 3 groups for the nibble and int8 containers, 2 for BF6 (whose conversion needs 16 more
// registers).  Larger ranks (LoRA adapters) hold more low-rank operands and accumulators
// (<= 256 VGPRs): batches of 6 groups, from rank 96 on batches of 3, and from rank 112 on
// batches of 2 (rank 128 still spills 4 to 25 dwords, by container).
constexpr int act_max_waves(int) { return 8; }
// Balanced grid (long K): when the row blocks outnumber the CUs but not twice over, one
// workgroup of 16 waves per CU takes an equal share of the (row block, group) units (ranks up
// to 32: at most 120 VGPRs, so 16 waves fit a CU).
constexpr int kActWideWaves = 16;
constexpr int kActShareSegs = 3;  // row blocks a share of at most 2 G units can span
constexpr int act_batch(int ntr, int codes) {
  return (codes == kCodesBf6 && ntr <= 2) || ntr >= 7 ? 2 : ntr <= 2 || ntr >= 6 ? 3 : 6;
}
constexpr size_t kActLdsLambda = 96 * 1024;  // inv_lambda staged in LDS while it fits

// max over the four lanes of a quad (one row): DPP quad permutations [1, 0, 3, 2] and
// [2, 3, 0, 1] bring each lane its neighbours' values within the VALU.
__device__ __forceinline__ float max_row_quarters(float a) {
  const float b = __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(a), 0xB1, 0xF, 0xF, false));
  a = __builtin_fmaxf(a, b);
  const float c = __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(a), 0x4E, 0xF, 0xF, false));
  return __builtin_fmaxf(a, c);
}

// the fixed lane permutation into the MFMA operand layout: each lane takes the dwords of the
// lane whose byte address src_byte gives (4 (4 (l % 16) + l / 16) for lane l)
__device__ __forceinline__ v4u quad_to_mfma(v4u v, int src_byte) {
  return v4u{(uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.x),
             (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.y),
             (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.z),
             (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.w)};
}

// A unit of work: row block rb (16 rows) x 64-group g, u = rb G + g.
struct ActUnit {
  int u, rb, g;
};

// CODES: kCodesNibbles, kCodesBf6 (INT4 codes) or kCodesInt8 (8-bit codes of the W4A8 variant)
// WAVES: the most waves a workgroup is launched with (the register budget follows from it);
// kActWideWaves is the balanced grid, whose shares span several row blocks (SHARE), and 8 the
// grid of one or two workgroups per row block
template <int NTR, int CODES, bool LAM_LDS, int WAVES>  // NTR: 16-wide tiles of the rank r = 16 NTR
__global__ __launch_bounds__(64 * WAVES) void quantize_act_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ inv_lambda,
    const uint16_t* __restrict__ L1, int M, int K, uint8_t* __restrict__ xq,
    uint16_t* __restrict__ x_scales, float* __restrict__ T, int nrb, int tadd) {
  // [K] inv_lambda (when staged), then the partial T slots [segments][nwaves][16][r]
  extern __shared__ float smem[];
  constexpr int r = 16 * NTR;
  constexpr int NT = NTR > 0 ? NTR : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int rl = lane >> 2;  // this lane's row of the block
  const int q = lane & 3;    // and quarter of the group
  const int src_byte = 4 * (4 * (lane & 15) + (lane >> 4));  // the MFMA layout's source lane
  const int G = K / kGroup;
  constexpr bool SHARE = WAVES == kActWideWaves;
  // The workgroup's share: units [u_lo, u_hi) of the nrb G units, split evenly over the grid.
  // One workgroup per row block (u_lo = rb G), two per row block (its halves, long K), or an
  // even share of at least G units per workgroup (more row blocks than CUs).  A share of at
  // least G units meets a row block's G units in at most two shares, so a row block's T is
  // either written by its one workgroup, or the sum of two partials added atomically onto a
  // zeroed T (the first addition is exact and fl32(a + b) = fl32(b + a): deterministic).  A
  // share of at most 2 G units spans at most three row blocks (kActShareSegs partial T slots).
  const long long U = (long long)nrb * G;
  const int u_lo = (int)((long long)blockIdx.x * U / gridDim.x);
  const int u_hi = (int)((long long)(blockIdx.x + 1) * U / gridDim.x);
  const int rb_first = u_lo / G;
  const ActUnit last{u_hi - 1, (u_hi - 1) / G, (u_hi - 1) % G};
  auto unit = [&](int u) { return ActUnit{u, u / G, u % G}; };
  // the wave's units are u_lo + wave + k nwaves; a unit past the share is clamped to the last
  // one (a clamped duplicate is computed but neither stored nor accumulated)
  auto clamp_unit = [&](const ActUnit& p) { return p.u < u_hi ? p : last; };
  // (one row block per share: the row block never changes, and a unit past it is clamped)
  auto advance = [&](ActUnit& p) {
    p.u += nwaves;
    p.g += nwaves;
    if constexpr (SHARE) {
      while (p.g >= G) {
        p.g -= G;
        ++p.rb;
      }
    }
  };
  auto row_block = [&](const ActUnit& p) { return SHARE ? p.rb : rb_first; };
  auto xptr = [&](const ActUnit& p) {
    const int rw = min(row_block(p) * kActRows + rl, M - 1);
    return reinterpret_cast<const v4u*>(X + (size_t)rw * K + (size_t)p.g * kGroup + 16 * q);
  };
  float* lam = smem;
  float* red = smem + (LAM_LDS ? K : 0);

  constexpr int kActBatch = act_batch(NTR, CODES);
  // Rolling pipeline over the wave's units: slot b of raw holds the activations of the batch's
  // unit b, and is refilled with unit b of the next batch as soon as it has been read, so the
  // next batch's loads are in flight under this batch's work.  The first batch is requested
  // before inv_lambda is staged, so the two round trips overlap.
  v4u raw[kActBatch][2];
  ActUnit fill = unit(u_lo + wave);  // the unit whose activations are loaded next
#pragma unroll
  for (int b = 0; b < kActBatch; ++b) {
    const v4u* p = xptr(clamp_unit(fill));
    raw[b][0] = p[0];
    raw[b][1] = p[1];
    advance(fill);
  }

  // inv_lambda is shared by every row: one coalesced copy into LDS per workgroup, so the group
  // loop's only global loads are the activations and L1, and no wait on them also waits for
  // the code stores (which count in the same counter)
  if constexpr (LAM_LDS) {
    for (int i = threadIdx.x; i < K / 4; i += blockDim.x)
      reinterpret_cast<v4f*>(lam)[i] = reinterpret_cast<const v4f*>(inv_lambda)[i];
  }
  // with several row blocks per share, a wave may meet only some of them: its other partial
  // T slots stay zero
  if constexpr (SHARE && NTR > 0)
    for (int i = threadIdx.x; i < kActShareSegs * nwaves * 16 * r; i += blockDim.x) red[i] = 0.0f;
  if constexpr (LAM_LDS || (SHARE && NTR > 0)) __syncthreads();

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // this lane's L1 values for group g (k = 16 q .. 16 q + 15 of rank rows 16 t + rl), in the
  // load layout
  auto load_l1 = [&](int g, v4u (&dst)[NT][2]) {
    if constexpr (NTR > 0) {
#pragma unroll
      for (int t = 0; t < NTR; ++t) {
        const v4u* bp = reinterpret_cast<const v4u*>(L1 + (size_t)(16 * t + rl) * K + (size_t)g * kGroup + 16 * q);
        dst[t][0] = bp[0];
        dst[t][1] = bp[1];
      }
    }
  };

  // this wave's partial T (acc) belongs to row block rb_acc; it moves to slot
  // rb_acc - rb_first of the wave when the wave's units pass into the next row block
  auto flush = [&](int rb) {
    if constexpr (NTR > 0) {
      // D layout of a 16x16 MFMA tile: lane l holds column l % 16 and rows 4 (l / 16) + i.
      float* slot = red + ((size_t)(rb - rb_first) * nwaves + wave) * 16 * r;
#pragma unroll
      for (int t = 0; t < NTR; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) slot[(4 * (lane >> 4) + i) * r + t * 16 + (lane & 15)] = acc[t][i];
    }
  };

  // L1 operands, one unit ahead of their use along the wave's whole sequence of units (the
  // next batch's first unit is requested under this batch's last)
  ActUnit cur = unit(u_lo + wave);  // the unit computed next
  int rb_acc = row_block(clamp_unit(cur));
  v4u bfr[2][NT][2];
  load_l1(clamp_unit(cur).g, bfr[0]);
  for (int j0 = u_lo + wave; j0 < u_hi; j0 += kActBatch * nwaves) {
    const bool more = j0 + kActBatch * nwaves < u_hi;  // uniform: this wave has a next batch
#pragma unroll
    for (int b = 0; b < kActBatch; ++b) {
      const bool gv = cur.u < u_hi;  // uniform over the wave
      const ActUnit cu = clamp_unit(cur);
      const int g = cu.g;
      const int row = row_block(cu) * kActRows + rl;
      advance(cur);
      if (b + 1 < kActBatch || more) load_l1(clamp_unit(cur).g, bfr[(b + 1) & 1]);
      const int k0 = g * kGroup + 16 * q;
      v4f l0, l1, l2, l3;
      if constexpr (LAM_LDS) {
        const v4f* lp = reinterpret_cast<const v4f*>(lam + k0);
        l0 = lp[0]; l1 = lp[1]; l2 = lp[2]; l3 = lp[3];
      } else {
        const v4f* lp = reinterpret_cast<const v4f*>(inv_lambda + k0);
        l0 = lp[0]; l1 = lp[1]; l2 = lp[2]; l3 = lp[3];
      }
      float xh[16];
      {
        const v4u w0 = raw[b][0], w1 = raw[b][1];
        xh[0] = __uint_as_float(w0.x << 16) * l0.x;
        xh[1] = __uint_as_float(w0.x & 0xFFFF0000u) * l0.y;
        xh[2] = __uint_as_float(w0.y << 16) * l0.z;
        xh[3] = __uint_as_float(w0.y & 0xFFFF0000u) * l0.w;
        xh[4] = __uint_as_float(w0.z << 16) * l1.x;
        xh[5] = __uint_as_float(w0.z & 0xFFFF0000u) * l1.y;
        xh[6] = __uint_as_float(w0.w << 16) * l1.z;
        xh[7] = __uint_as_float(w0.w & 0xFFFF0000u) * l1.w;
        xh[8] = __uint_as_float(w1.x << 16) * l2.x;
        xh[9] = __uint_as_float(w1.x & 0xFFFF0000u) * l2.y;
        xh[10] = __uint_as_float(w1.y << 16) * l2.z;
        xh[11] = __uint_as_float(w1.y & 0xFFFF0000u) * l2.w;
        xh[12] = __uint_as_float(w1.z << 16) * l3.x;
        xh[13] = __uint_as_float(w1.z & 0xFFFF0000u) * l3.y;
        xh[14] = __uint_as_float(w1.w << 16) * l3.z;
        xh[15] = __uint_as_float(w1.w & 0xFFFF0000u) * l3.w;
      }
      if (more) {  // refill slot b with unit b of the next batch
        const v4u* p = xptr(clamp_unit(fill));
        raw[b][0] = p[0];
        raw[b][1] = p[1];
      }
      advance(fill);

      // ---- group max over the row's four quarter lanes, scale, codes
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[i]));
      amax = max_row_quarters(amax);
      constexpr bool I8 = CODES == kCodesInt8;
      const uint16_t sb = I8 ? int8_scale_bits(amax) : int4_scale_bits(amax);
      const float s = half_bits_to_float(sb);
      const float s1 = s == 0.0f ? 1.0f : s;  // an all-zero group: every quotient is 0
      const bool live = row < M;
      // padding rows get 1 / s = 0: every quotient is then exactly 0, so no select per code
      const float rcp = live ? rcp_rn_half(s1) : 0.0f;
      // code + 8 (+ 128 for 8-bit codes) as bytes: rne of the correctly rounded quotient, the
      // bias, clamp to [0, 15] ([0, 255]); a -0 quotient becomes the bias, so both zeros give 0
      constexpr float kBias = I8 ? 128.0f : 8.0f, kTop = I8 ? 255.0f : 15.0f;
      uint32_t bq[4];
      if constexpr (CODES == kCodesBf6) {
        // BF6 container: the codes as floats (-0 made +0, clamped to [-8, 7]) go through the
        // hardware fp32 -> BF6 conversion, which packs 2 x 16 values with value 2i from the
        // first source and 2i + 1 from the second, 6 bits each: the even and odd codes of the
        // group give its 16 codes in order in the first three dwords (every integer in
        // [-8, 7] is an exact E3M2 value, so the conversion only re-encodes).
        // (elements 8..15 of each source are left undefined: they only feed output dwords 3..5,
        // which are not stored)
        v16f ce, co;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ce[i] = __builtin_amdgcn_fmed3f(rne_quotient(xh[2 * i], s1, rcp) + 0.0f, -8.0f, 7.0f);
          co[i] = __builtin_amdgcn_fmed3f(rne_quotient(xh[2 * i + 1], s1, rcp) + 0.0f, -8.0f, 7.0f);
        }
        // The conversion writes its first result dword before it has read every source
        // element, and the compiler's builtin may give it a destination that overlaps a source
        // (seen: destination v[6:11] over the first source's element 4, which then read back
        // as the result's first dword).  So it is issued here with an early-clobber
        // destination, disjoint from both sources, and followed by wait states before any use
        // of its result.
        v6u w6;
        asm("v_cvt_scalef32_2xpk16_bf6_f32 %0, %1, %2, 1.0\n\ts_nop 7"
                     : "=&v"(w6)
                     : "v"(ce), "v"(co));
        if (gv) {  // rows up to the block boundary (padding rows: zero codes)
          uint8_t* dst = xq + ((size_t)(row >> 5) * G + g) * kE3m2Block + ((row & 31) + 32 * (q >> 1)) * 24 + 12 * (q & 1);
          *reinterpret_cast<v3u*>(dst) = v3u{w6[0], w6[1], w6[2]};
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_fmed3f(rne_quotient(xh[4 * d + i], s1, rcp) + kBias, 0.0f, kTop);
          bq[d] = bytes4(v);
        }
      }
      if (gv) {
        if (live) {
          if constexpr (CODES == kCodesNibbles)
            *reinterpret_cast<v2u*>(xq + (size_t)row * (K / 2) + (size_t)g * 32 + 8 * q) = v2u{nibbles8_biased(bq[0], bq[1]), nibbles8_biased(bq[2], bq[3])};
          if constexpr (I8)  // c + 128 xor 128 is the two's complement byte of c
            *reinterpret_cast<v4u*>(xq + (size_t)row * K + (size_t)g * kGroup + 16 * q) =
                v4u{bq[0], bq[1], bq[2], bq[3]} ^ 0x80808080u;
          if (q == 0) x_scales[(size_t)row * G + g] = sb;  // [M, G]
        }
      }

      // ---- low-rank down-projection on bf16 MFMA (a clamped duplicate unit adds zero)
      if constexpr (NTR > 0) {
        if constexpr (SHARE) {
          if (gv && cu.rb != rb_acc) {  // uniform: the wave passes into the next row block
            flush(rb_acc);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
            rb_acc = cu.rb;
          }
        }
        v8bf a0 = __builtin_bit_cast(v8bf, quad_to_mfma(__builtin_bit_cast(v4u, to_bf16x8(xh)), src_byte));
        v8bf a1 = __builtin_bit_cast(v8bf, quad_to_mfma(__builtin_bit_cast(v4u, to_bf16x8(xh + 8)), src_byte));
        if (!gv) a0 = a1 = v8bf{};
#pragma unroll
        for (int t = 0; t < NTR; ++t) {
          const v8bf b0 = __builtin_bit_cast(v8bf, quad_to_mfma(bfr[b & 1][t][0], src_byte));
          const v8bf b1 = __builtin_bit_cast(v8bf, quad_to_mfma(bfr[b & 1][t][1], src_byte));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[t], 0, 0, 0);
        }
      }
    }
    // an odd batch leaves the next batch's first operands in slot 1; group 0 reads slot 0
    if constexpr (kActBatch % 2 == 1 && NTR > 0) {
#pragma unroll
      for (int t = 0; t < NTR; ++t) {
        bfr[0][t][0] = bfr[1][t][0];
        bfr[0][t][1] = bfr[1][t][1];
      }
    }
  }

  if constexpr (NTR > 0) {
    flush(rb_acc);
    __syncthreads();
    // each row block's partial: the waves' partials summed in wave order
    const int nused = last.rb - rb_first + 1;
    for (int idx = threadIdx.x; idx < nused * 16 * r; idx += blockDim.x) {
      const int sg = idx / (16 * r), within = idx - sg * 16 * r;
      const float* slots = red + (size_t)sg * nwaves * 16 * r + within;
      float sum = 0.0f;
      for (int w = 0; w < nwaves; ++w) sum += slots[(size_t)w * 16 * r];
      const int rw = (rb_first + sg) * kActRows + within / r;
      if (rw < M) {
        float* t = T + (size_t)rw * r + (within % r);
        if (tadd)
          atomicAdd(t, sum);
        else
          *t = sum;
      }
    }
  }
}

template <int CODES, bool LAM_LDS, int WAVES>
static hipError_t launch_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                             int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                             int nrb, int grid, int nwaves, int tadd, size_t lds,
                             hipStream_t stream) {
  switch (r / 16) {
#define SVDQ_ACT_CASE(n)                                                                     \
  case n: {                                                                                  \
    if constexpr (WAVES <= act_max_waves(n) || n <= 2) { /* 16 waves: rank <= 32 */       \
      const void* fn = reinterpret_cast<const void*>(quantize_act_kernel<n, CODES, LAM_LDS, WAVES>); \
      if (lds > 64 * 1024) {                                                                 \
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e;                                                       \
      }                                                                                      \
      hipLaunchKernelGGL((quantize_act_kernel<n, CODES, LAM_LDS, WAVES>), dim3(grid),       \
                         dim3(64 * nwaves), lds, stream, X, inv_lambda, L1, M, K, xq, x_scales, \
                         T, nrb, tadd);                                                      \
      break;                                                                                 \
    } else {                                                                                 \
      return hipErrorInvalidValue;                                                           \
    }                                                                                        \
  }
    SVDQ_ACT_CASE(0)
    SVDQ_ACT_CASE(1)
    SVDQ_ACT_CASE(2)
    SVDQ_ACT_CASE(3)
    SVDQ_ACT_CASE(4)
    SVDQ_ACT_CASE(5)
    SVDQ_ACT_CASE(6)
    SVDQ_ACT_CASE(7)
    SVDQ_ACT_CASE(8)
#undef SVDQ_ACT_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// zeroes T ahead of a pass whose row blocks are shared by two workgroups (a fill kernel, not
// a memset, so that the call can be captured in a graph)
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0.0f;
}

// Groups per row block from which the pass splits K: with long K a row block's workgroup runs
// long enough that the row blocks past one per CU double their CUs' time.  Up to one row
// block per CU each row block's halves go to two workgroups; with more (but fewer than two per
// CU), the balanced grid gives every CU an equal share.  FFN down (K = 12288, rank 32): 4096
// tokens took 46.9 us with one workgroup per row block; 4608 tokens 75 us, 64 us in halves,
// 55.8 us on the balanced grid.  At shorter K the balanced grid lost (4608 x 3072: 18.4 ->
// 22.0 us; the fill of T and the shares' partial sums cost more than the balance saves).
constexpr int kActSplitGroups = 96;

// the current device's CU count and largest LDS allocation per workgroup (0 if unknown)
struct ActDevice {
  int cus, lds;
};
static ActDevice act_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<long long> cache[kMaxDevices];  // cus << 32 | lds, + 1; 0 = not queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return {0, 0};
  }
  const long long c = cache[dev].load(std::memory_order_relaxed);
  if (c) return {(int)((c - 1) >> 32), (int)((c - 1) & 0xFFFFFFFF)};
  int cus = 0, lds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error behind; use the per-row-block grid
    return {0, 0};
  }
  cache[dev].store((((long long)cus << 32) | (unsigned)lds) + 1, std::memory_order_relaxed);
  return {cus, lds};
}

template <int CODES>
static hipError_t launch_act_route(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                                   int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                                   hipStream_t stream) {
  const int G = K / kGroup;
  // the tiled BF6 container is written up to the next multiple of 32 rows
  const int rows = CODES == kCodesBf6 ? (M + kE3m2Rows - 1) / kE3m2Rows * kE3m2Rows : M;
  const int nrb = (rows + kActRows - 1) / kActRows;
  const size_t lam = (size_t)K * sizeof(float);
  // Balanced grid (long K, between one and two row blocks per CU, rank <= 32): one workgroup
  // of 16 waves per CU, each with an even share of the units (at least G and at most 2 G).
  const ActDevice dev = act_device();
  static_assert(kActSplitGroups >= kActWideWaves, "a wave's next unit is at most one row block on");
  if (r <= 32 && G >= kActSplitGroups && dev.cus > 0 && nrb > dev.cus && nrb < 2 * dev.cus) {
    const size_t red = (size_t)kActShareSegs * kActWideWaves * 16 * r * sizeof(float);
    if (red <= (size_t)dev.lds) {
      if (r > 0) {
        const size_t n = (size_t)M * r;
        const size_t want = (n + 255) / 256;
        hipLaunchKernelGGL(zero_f32_kernel, dim3(want < 4096 ? (int)want : 4096), dim3(256), 0,
                           stream, T, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      if (lam + red <= (size_t)dev.lds)
        return launch_act<CODES, true, kActWideWaves>(X, inv_lambda, L1, M, K, r, xq, x_scales, T,
                                                      nrb, dev.cus, kActWideWaves, 1, lam + red,
                                                      stream);
      return launch_act<CODES, false, kActWideWaves>(X, inv_lambda, L1, M, K, r, xq, x_scales, T,
                                                     nrb, dev.cus, kActWideWaves, 1, red, stream);
    }
  }
  // one workgroup per row block, or two (its halves) from kActSplitGroups groups on
  const int ksplit = G >= kActSplitGroups ? 1 : 0;
  const int Gw = ksplit ? (G + 1) / 2 : G;  // groups per workgroup
  const int maxw = act_max_waves(r / 16);
  const int nwaves = Gw < maxw ? Gw : maxw;
  if (ksplit && r > 0) {
    const size_t n = (size_t)M * r;
    const size_t want = (n + 255) / 256;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(want < 4096 ? (int)want : 4096), dim3(256), 0, stream,
                       T, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t red = (size_t)nwaves * 16 * r * sizeof(float);
  const int grid = nrb << ksplit;
  if (lam + red <= kActLdsLambda)
    return launch_act<CODES, true, 8>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, nrb, grid,
                                      nwaves, ksplit, lam + red, stream);
  return launch_act<CODES, false, 8>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, nrb, grid, nwaves,
                                     ksplit, red, stream);
}

hipError_t launch_quantize_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                               int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                               int codes, hipStream_t stream) {
  switch (codes) {
    case kCodesNibbles:
      return launch_act_route<kCodesNibbles>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, stream);
    case kCodesBf6:
      return launch_act_route<kCodesBf6>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, stream);
    case kCodesInt8:
      return launch_act_route<kCodesInt8>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace svdq
