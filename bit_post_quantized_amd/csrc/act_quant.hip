// Fused activation pass: smoothing, dynamic low-bit quantization and the low-rank
// down-projection.
//
// SVDQ "technical principles": smoothing moves activation outliers into the weights, and a
// 16-bit low-rank branch runs beside the 4-bit one.  FLUX4 3.1: activations are quantized at
// run time.  W4A8 3.1: symmetric scale max|v| / (2^(b-1) - 1), round, clamp, one scale per
// token and 64-group; b = 4 (INT4 codes) or b = 8 (the W4A8 variant's activations, W4A8 1).
// SVDQ / DCMP: the branch is fused so the activations are read from HBM once.
//
// Work decomposition.  A workgroup owns 16 tokens (rows) and all of K; its waves take the
// 64-groups round-robin.  In a group, lane l holds row l / 4 and the 16 consecutive k
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
// Per-wave partial T tiles are summed in LDS in wave order (deterministic) and written once.
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
// (<= 256 VGPRs): batches of 6 groups, and from rank 96 on, batches of 3 (no spills at any
// rank).
constexpr int act_max_waves(int) { return 8; }
constexpr int act_batch(int ntr, int codes) {
  return codes == kCodesBf6 && ntr <= 2 ? 2 : ntr <= 2 || ntr >= 6 ? 3 : 6;
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

// CODES: kCodesNibbles, kCodesBf6 (INT4 codes) or kCodesInt8 (8-bit codes of the W4A8 variant)
template <int NTR, int CODES, bool LAM_LDS>  // NTR: 16-wide tiles of the rank r (r = 16 * NTR)
__global__ __launch_bounds__(64 * act_max_waves(NTR)) void quantize_act_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ inv_lambda,
    const uint16_t* __restrict__ L1, int M, int K, uint8_t* __restrict__ xq,
    uint16_t* __restrict__ x_scales, float* __restrict__ T, int ksplit) {
  extern __shared__ float smem[];  // [K] inv_lambda (when staged), then [nwaves][16][r]
  constexpr int r = 16 * NTR;
  constexpr int NT = NTR > 0 ? NTR : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int rl = lane >> 2;  // this lane's row of the block
  const int q = lane & 3;    // and quarter of the group
  const int src_byte = 4 * (4 * (lane & 15) + (lane >> 4));  // the MFMA layout's source lane
  const int G = K / kGroup;
  // K split (long K): two neighbouring workgroups take the two halves of a row block's groups;
  // their partial T meet by two atomic additions onto a zeroed T (exact for the first, and the
  // same for either order: fl32(a + b) = fl32(b + a)), so the result is deterministic
  const int half = ksplit ? (int)(blockIdx.x & 1) : 0;
  const int Gh = (G + 1) / 2;
  const int g_lo = ksplit ? half * Gh : 0;
  const int g_hi = ksplit ? min(G, g_lo + Gh) : G;
  const int row0 = (ksplit ? (int)(blockIdx.x >> 1) : (int)blockIdx.x) * kActRows;
  const int row = row0 + rl;
  const int row_ld = row < M ? row : M - 1;
  const uint16_t* xrow = X + (size_t)row_ld * K + 16 * q;
  float* lam = smem;
  float* red = smem + (LAM_LDS ? K : 0);

  constexpr int kActBatch = act_batch(NTR, CODES);
  // Rolling pipeline over the wave's groups j0 + b nwaves: slot b of raw holds the activations
  // of the batch's group b, and is refilled with group b of the next batch as soon as it has
  // been read, so the next batch's loads are in flight under this batch's work (group index
  // clamped; a clamped duplicate is computed but neither stored nor accumulated).  The first
  // batch is requested before inv_lambda is staged, so the two round trips overlap.
  v4u raw[kActBatch][2];
#pragma unroll
  for (int b = 0; b < kActBatch; ++b) {
    const int g = min(g_lo + wave + b * nwaves, g_hi - 1);
    const v4u* p = reinterpret_cast<const v4u*>(xrow + (size_t)g * kGroup);
    raw[b][0] = p[0];
    raw[b][1] = p[1];
  }

  // inv_lambda is shared by every row: one coalesced copy into LDS per workgroup, so the group
  // loop's only global loads are the activations and L1, and no wait on them also waits for
  // the code stores (which count in the same counter)
  if constexpr (LAM_LDS) {
    for (int i = threadIdx.x; i < K / 4; i += blockDim.x)
      reinterpret_cast<v4f*>(lam)[i] = reinterpret_cast<const v4f*>(inv_lambda)[i];
    __syncthreads();
  }

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

  // L1 operands, one group ahead of their use along the wave's whole sequence of groups (the
  // next batch's first group is requested under this batch's last)
  v4u bfr[2][NT][2];
  load_l1(min(g_lo + wave, g_hi - 1), bfr[0]);
  for (int j0 = g_lo + wave; j0 < g_hi; j0 += kActBatch * nwaves) {
    const bool more = j0 + kActBatch * nwaves < g_hi;  // uniform: this wave has a next batch
#pragma unroll
    for (int b = 0; b < kActBatch; ++b) {
      const int g_raw = j0 + b * nwaves;
      const bool gv = g_raw < g_hi;  // uniform over the wave
      const int g = gv ? g_raw : g_hi - 1;
      if (b + 1 < kActBatch || more) load_l1(min(j0 + (b + 1) * nwaves, g_hi - 1), bfr[(b + 1) & 1]);
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
      if (more) {  // refill slot b with group b of the next batch
        const int gn = min(j0 + (kActBatch + b) * nwaves, g_hi - 1);
        const v4u* p = reinterpret_cast<const v4u*>(xrow + (size_t)gn * kGroup);
        raw[b][0] = p[0];
        raw[b][1] = p[1];
      }

      // ---- group max over the row's four quarter lanes, scale, codes
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[i]));
      amax = max_row_quarters(amax);
      constexpr bool I8 = CODES == kCodesInt8;
      const uint16_t sb = I8 ? float_to_half_bits(amax / 127.0f) : int4_scale_bits(amax);
      const float s = half_bits_to_float(sb);
      const float s1 = s == 0.0f ? 1.0f : s;  // an all-zero group: every quotient is 0
      const bool live = row < M;
      // padding rows get 1 / s = 0: every quotient is then exactly 0, so no select per code
      const float rcp = live ? 1.0f / s1 : 0.0f;
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

      // ---- low-rank down-projection on bf16 MFMA (a clamped duplicate group adds zero)
      if constexpr (NTR > 0) {
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
    // D layout of a 16x16 MFMA tile: lane l holds column l % 16 and rows 4 * (l / 16) + i.
#pragma unroll
    for (int t = 0; t < NTR; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[((size_t)wave * 16 + 4 * (lane >> 4) + i) * r + t * 16 + (lane & 15)] = acc[t][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * r; idx += blockDim.x) {
      const int rr = idx / r;
      float sum = 0.0f;
      for (int w = 0; w < nwaves; ++w) sum += red[(size_t)w * 16 * r + idx];
      if (row0 + rr < M) {
        float* t = T + (size_t)(row0 + rr) * r + (idx % r);
        if (ksplit)
          atomicAdd(t, sum);
        else
          *t = sum;
      }
    }
  }
}

template <int CODES, bool LAM_LDS>
static hipError_t launch_act(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                             int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                             int nwaves, size_t lds, int ksplit, hipStream_t stream) {
  // the tiled BF6 container is written up to the next multiple of 32 rows
  const int rows = CODES == kCodesBf6 ? (M + kE3m2Rows - 1) / kE3m2Rows * kE3m2Rows : M;
  const dim3 grid(((rows + kActRows - 1) / kActRows) << ksplit), block(64 * nwaves);
  switch (r / 16) {
#define SVDQ_ACT_CASE(n)                                                                   \
  case n: {                                                                                \
    const void* fn = reinterpret_cast<const void*>(quantize_act_kernel<n, CODES, LAM_LDS>);  \
    if (lds > 64 * 1024) {                                                                 \
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e != hipSuccess) return e;                                                       \
    }                                                                                      \
    hipLaunchKernelGGL((quantize_act_kernel<n, CODES, LAM_LDS>), grid, block, lds, stream, X, \
                       inv_lambda, L1, M, K, xq, x_scales, T, ksplit);                     \
    break;                                                                                 \
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

// zeroes T ahead of a K-split pass (a fill kernel, not a memset, so that the call can be
// captured in a graph)
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0.0f;
}

// Groups per row block from which the pass splits K over two workgroups: with long K a row
// block's workgroup runs long enough that the row blocks past one per CU (288 on 256 CUs at
// 4608 tokens) double their CUs' time; halves balance that (FFN down, K = 12288: 4096 tokens
// took 46.9 us, 4608 tokens 75 us).
constexpr int kActSplitGroups = 96;

template <int CODES>
static hipError_t launch_act_route(const uint16_t* X, const float* inv_lambda, const uint16_t* L1,
                                   int M, int K, int r, uint8_t* xq, uint16_t* x_scales, float* T,
                                   hipStream_t stream) {
  const int G = K / kGroup;
  const int ksplit = G >= kActSplitGroups ? 1 : 0;
  const int Gw = ksplit ? (G + 1) / 2 : G;  // groups per workgroup
  const int maxw = act_max_waves(r / 16);
  const int nwaves = Gw < maxw ? Gw : maxw;
  if (ksplit && r > 0 && M > 0) {
    const size_t n = (size_t)M * r;
    const size_t want = (n + 255) / 256;
    const int blocks = want < 4096 ? (int)want : 4096;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(256), 0, stream, T, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t red = (size_t)nwaves * 16 * r * sizeof(float);
  const size_t lam = (size_t)K * sizeof(float);
  if (lam + red <= kActLdsLambda)
    return launch_act<CODES, true>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, nwaves, lam + red,
                                   ksplit, stream);
  return launch_act<CODES, false>(X, inv_lambda, L1, M, K, r, xq, x_scales, T, nwaves, red, ksplit,
                                  stream);
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
