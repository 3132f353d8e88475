// W4A4 group GEMM on the FP6 matrix units: the INT4 codes of both operands are carried as BF6
// (E3M2) values, with the low-rank up-projection and bias fused into the epilogue.
//
// Same result as the INT8-unit GEMM (SVDQ "technical principles"; DCMP "SVDQuant" section):
//     Y = sum_g diag(s_x[g]) P[g] diag(s_w[g]) + bf16(T) L2 + bias,
//     P[g] = qx[:, g] . qw[g, :]   (exact).
// FLUX4 3.2 notes that a small floating-point format read directly by the matrix units avoids
// the 4-bit unpack that INT4 needs on INT8 units (W4A8 2.2).  On gfx950 that format is BF6:
// every code in [-8, 8] is an exact E3M2 value, so v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales (E8M0 127) returns the 32 x 32 partial of one 64-group exactly in fp32
// (integers of magnitude <= 4096), at twice the FP8 / INT8 rate, and no int -> float convert
// is left in the dequantization.
//
// gfx950 mapping (one workgroup = 4 waves = a 128 x 128 tile of Y; wave (wm, wn) owns the
// 64 x 64 sub-tile made of 2 x 2 tiles of 32 x 32):
//  * MFMA operand layout (32 x 32 x 64 f8f6f4, BF6): lane l supplies row (or column) l % 32 and
//    the 32 codes k = 32 (l / 32) + i as six dwords, code i at bits 6i .. 6i+5 -- exactly half
//    of a group's 48-byte record in the packed stream.  The 32 x 32 result: lane l holds column
//    l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4, e = 0..15.
//  * Staging.  KS = 2 groups per stage.  Thread t copies the two 24-byte halves of one
//    (row, group) record (three 16-byte global loads) into "lane slots": for every 32-row tile
//    and group, 64 consecutive 24-byte slots in MFMA lane order, so a fragment is three
//    conflict-free ds_read_b64 per lane.  Two LDS buffers alternate; the next stage's global
//    loads are in flight while the current one is computed; one barrier per stage.
//  * Scale products.  s_x[m] * s_w[n] for a 32 x 32 tile is an outer product that
//    v_mfma_f32_32x32x8_f16 computes exactly (fp16 x fp16 is exact in fp32) when only k-slot 0
//    is nonzero: the scales sit in LDS slots 0..31 and slots 32..63 hold zeros, so every lane's
//    operand is one ds_read_u16.  The dequantization is one FMA per output and group.
//  * Epilogue.  bf16(T) [32 x 16] and L2 [16 x 32] fragments go through
//    v_mfma_f32_32x32x16_bf16 with the fp32 accumulator as C, then the bias is added and the
//    tile is rounded to bf16 (or kept fp32) and stored.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

namespace f6 {
constexpr int kRecord = 48;                         // one 64-group of one row: 64 x 6 bits
constexpr int kSlot = 24;                           // one lane's half of a record
constexpr int kBlock = 64 * kSlot + 16;             // 64 lane slots (+16 bytes against bank aliasing)
constexpr int TM = 128, TN = 128;                   // workgroup tile
constexpr int KS = 2;                               // groups per LDS stage
constexpr int THREADS = 256;                        // 2 x 2 waves of 64 x 64
constexpr int RT = TM / 32, CT = TN / 32;           // 32 x 32 tiles along M and N
constexpr int kOpA = RT * KS * kBlock;
constexpr int kOpB = CT * KS * kBlock;
constexpr int kScA = KS * RT * 64 * 2;              // fp16 [KS][RT][64 slots]
constexpr int kScB = KS * CT * 64 * 2;
constexpr int kStage = kOpA + kOpB + kScA + kScB;
constexpr int kLds = 2 * kStage;
static_assert(TM * KS == THREADS && TN * KS == THREADS, "one record per thread and operand");
static_assert(KS * TM == THREADS && KS * TN == THREADS, "one scale per thread and operand");
static_assert(kBlock % 16 == 0 && kStage % 16 == 0, "16-byte aligned LDS areas");
}  // namespace f6

template <bool OUT_FP32, bool PARTIALS, int NTR>
__global__ __launch_bounds__(f6::THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void w4a4_gemm_e3m2_kernel(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ x_scales,
    const float* __restrict__ T, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ w_scales, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, int M, int N, int K, void* __restrict__ Y,
    int32_t* __restrict__ P) {
  using namespace f6;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int r = 16 * NTR;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m_tile = blockIdx.y * TM, n_tile = blockIdx.x * TN;
  const int G = K / kGroup;
  const size_t ldq = (size_t)K / 4 * 3;

  // ---- staging map: thread t moves record (row t / KS, group t % KS) of A and of B, and the
  //      scale of (group t / TM, row t % TM) of s_x and of (group t / TN, column t % TN) of s_w
  const int u_row = tid / KS, u_g = tid % KS;
  const uint8_t* a_src = xq + (size_t)min(m_tile + u_row, M - 1) * ldq;
  const uint8_t* b_src = wq + (size_t)min(n_tile + u_row, N - 1) * ldq;
  const int a_dst = ((u_row >> 5) * KS + u_g) * kBlock + (u_row & 31) * kSlot;
  const int b_dst = kOpA + a_dst;
  const int s_g = tid / TM, s_r = tid % TM;
  const uint16_t* sx_src = PARTIALS ? nullptr : x_scales + min(m_tile + s_r, M - 1);
  const uint16_t* sw_src = PARTIALS ? nullptr : w_scales + min(n_tile + s_r, N - 1);
  const int sx_dst = kOpA + kOpB + (s_g * RT + (s_r >> 5)) * 128 + (s_r & 31) * 2;
  const int sw_dst = kOpA + kOpB + kScA + (s_g * CT + (s_r >> 5)) * 128 + (s_r & 31) * 2;

  struct Regs {
    v4u a[3], b[3];
    uint32_t sx, sw;
  };
  auto load_stage = [&](int s, Regs& R) {
    const int g = min(s * KS + u_g, G - 1);
    const v4u* pa = reinterpret_cast<const v4u*>(a_src + (size_t)g * kRecord);
    const v4u* pb = reinterpret_cast<const v4u*>(b_src + (size_t)g * kRecord);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      R.a[c] = pa[c];
      R.b[c] = pb[c];
    }
    if constexpr (!PARTIALS) {
      const int gs = s * KS + s_g;
      const int gl = min(gs, G - 1);
      const uint32_t keep = gs < G ? 0xFFFFu : 0u;  // a group past the end gets zero scales
      R.sx = sx_src[(size_t)gl * M] & keep;
      R.sw = sw_src[(size_t)gl * N] & keep;
    }
  };
  auto store_stage = [&](int buf, const Regs& R) {
    uint8_t* st = lds + buf * kStage;
    v2u* a0 = reinterpret_cast<v2u*>(st + a_dst);
    v2u* a1 = reinterpret_cast<v2u*>(st + a_dst + 32 * kSlot);
    a0[0] = v2u{R.a[0].x, R.a[0].y};
    a0[1] = v2u{R.a[0].z, R.a[0].w};
    a0[2] = v2u{R.a[1].x, R.a[1].y};
    a1[0] = v2u{R.a[1].z, R.a[1].w};
    a1[1] = v2u{R.a[2].x, R.a[2].y};
    a1[2] = v2u{R.a[2].z, R.a[2].w};
    v2u* b0 = reinterpret_cast<v2u*>(st + b_dst);
    v2u* b1 = reinterpret_cast<v2u*>(st + b_dst + 32 * kSlot);
    b0[0] = v2u{R.b[0].x, R.b[0].y};
    b0[1] = v2u{R.b[0].z, R.b[0].w};
    b0[2] = v2u{R.b[1].x, R.b[1].y};
    b1[0] = v2u{R.b[1].z, R.b[1].w};
    b1[1] = v2u{R.b[2].x, R.b[2].y};
    b1[2] = v2u{R.b[2].z, R.b[2].w};
    if constexpr (!PARTIALS) {
      *reinterpret_cast<uint16_t*>(st + sx_dst) = (uint16_t)R.sx;
      *reinterpret_cast<uint16_t*>(st + sw_dst) = (uint16_t)R.sw;
    }
  };

  // ---- per-lane fragment offsets inside a stage
  const int a_frag = (2 * wm * KS) * kBlock + lane * kSlot;       // + (i * KS + gg) * kBlock
  const int b_frag = kOpA + (2 * wn * KS) * kBlock + lane * kSlot;
  const int sa_frag = kOpA + kOpB + (2 * wm) * 128 + lane * 2;     // + (gg * RT + i) * 128
  const int sb_frag = kOpA + kOpB + kScA + (2 * wn) * 128 + lane * 2;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const v16f zero16 = acc[0][0];

  // scale slots 32..63 of both buffers must read as zero; the staging never writes them
  if constexpr (!PARTIALS) {
    for (int o = tid * 16; o < kScA + kScB; o += THREADS * 16) {
      *reinterpret_cast<v4u*>(lds + kOpA + kOpB + o) = v4u{0u, 0u, 0u, 0u};
      *reinterpret_cast<v4u*>(lds + kStage + kOpA + kOpB + o) = v4u{0u, 0u, 0u, 0u};
    }
  }
  const int S = (G + KS - 1) / KS;
  Regs R;
  load_stage(0, R);
  __syncthreads();
  store_stage(0, R);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    if (s + 1 < S) load_stage(s + 1, R);
    const uint8_t* st = lds + (s & 1) * kStage;
    const int ng = min(KS, G - s * KS);
#pragma unroll
    for (int gg = 0; gg < KS; ++gg) {
      if (gg >= ng) break;  // uniform
      v8i A[2], B[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v2u* pa = reinterpret_cast<const v2u*>(st + a_frag + (i * KS + gg) * kBlock);
        const v2u* pb = reinterpret_cast<const v2u*>(st + b_frag + (i * KS + gg) * kBlock);
        const v2u a0 = pa[0], a1 = pa[1], a2 = pa[2];
        const v2u b0 = pb[0], b1 = pb[1], b2 = pb[2];
        A[i] = v8i{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
        B[i] = v8i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y, (int)b2.x, (int)b2.y, 0, 0};
      }
      if constexpr (PARTIALS) {
        const int g = s * KS + gg;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], zero16, 3, 3, 0, 127, 0, 127);
            const int col = n_tile + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = m_tile + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              if (row < M && col < N) P[((size_t)g * M + row) * N + col] = (int32_t)p[e];  // exact
            }
          }
      } else {
        v4h SA[2], SB[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t sx = *reinterpret_cast<const uint16_t*>(st + sa_frag + (gg * RT + i) * 128);
          const uint32_t sw = *reinterpret_cast<const uint16_t*>(st + sb_frag + (gg * CT + i) * 128);
          SA[i] = __builtin_bit_cast(v4h, v2u{sx, 0u});
          SB[i] = __builtin_bit_cast(v4h, v2u{sw, 0u});
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], zero16, 3, 3, 0, 127, 0, 127);
            const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(SA[i], SB[j], zero16, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(p[e], sp[e], acc[i][j][e]);
            // keep this tile's dequantization here instead of letting the optimizer sink every
            // FMA below the last MFMA (which would keep all MFMA results live at once)
            asm volatile("" : "+v"(acc[i][j]));
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    }
    if (s + 1 < S) store_stage((s + 1) & 1, R);
    __syncthreads();
  }
  if constexpr (PARTIALS) return;

  // ---- epilogue: low-rank up-projection, bias, store.  The addresses are loop-invariant;
  //      computed before the K loop they would stay live across it, so they go through an
  //      opaque copy here.
  int row0 = m_tile + wm * 64, col0 = n_tile + wn * 64, Mo = M, No = N;
  asm volatile("" : "+v"(row0), "+v"(col0), "+s"(Mo), "+s"(No));
  const int l32 = lane & 31, hi = lane >> 5;
  if constexpr (NTR > 0) {
#pragma unroll
    for (int kk = 0; kk < r; kk += 16) {
      const int k8 = kk + 8 * hi;  // this lane's 8 rank indices
      v8bf Bt[2], At[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        Bt[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(L2 + (size_t)min(col0 + 32 * j + l32, No - 1) * r + k8));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4f* tp = reinterpret_cast<const v4f*>(T + (size_t)min(row0 + 32 * i + l32, Mo - 1) * r + k8);
        const v4f t0 = tp[0], t1 = tp[1];
        const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
        At[i] = to_bf16x8(tv);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[i], Bt[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + 32 * j + l32;
    const float bj = bias ? bf16_bits_to_float(bias[min(col, No - 1)]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < Mo && col < No) {
          const float v = acc[i][j][e] + bj;
          if constexpr (OUT_FP32)
            reinterpret_cast<float*>(Y)[(size_t)row * No + col] = v;
          else
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * No + col] = float_to_bf16_bits(v);
        }
      }
  }
}

template <bool OUT_FP32, bool PARTIALS>
static hipError_t launch_e3m2_ntr(int ntr, dim3 grid, hipStream_t stream, const uint8_t* xq,
                                  const uint16_t* x_scales, const float* T, const uint8_t* wq,
                                  const uint16_t* w_scales, const uint16_t* L2,
                                  const uint16_t* bias, int M, int N, int K, void* Y,
                                  int32_t* P) {
  switch (ntr) {
#define SVDQ_E3M2_CASE(n)                                                                      \
  case n:                                                                                      \
    hipLaunchKernelGGL((w4a4_gemm_e3m2_kernel<OUT_FP32, PARTIALS, n>), grid, dim3(f6::THREADS), \
                       f6::kLds, stream, xq, x_scales, T, wq, w_scales, L2, bias, M, N, K, Y,   \
                       P);                                                                     \
    break;
    SVDQ_E3M2_CASE(0)
    SVDQ_E3M2_CASE(1)
    SVDQ_E3M2_CASE(2)
    SVDQ_E3M2_CASE(3)
    SVDQ_E3M2_CASE(4)
    SVDQ_E3M2_CASE(5)
    SVDQ_E3M2_CASE(6)
    SVDQ_E3M2_CASE(7)
    SVDQ_E3M2_CASE(8)
#undef SVDQ_E3M2_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm_e3m2(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                                 const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                                 const uint16_t* bias, int M, int N, int K, int r, void* Y,
                                 int out_fp32, int32_t* partials, hipStream_t stream) {
  const dim3 grid((N + f6::TN - 1) / f6::TN, (M + f6::TM - 1) / f6::TM);
  if (partials)
    return launch_e3m2_ntr<false, true>(0, grid, stream, xq, nullptr, nullptr, wq, nullptr,
                                        nullptr, nullptr, M, N, K, nullptr, partials);
  if (out_fp32)
    return launch_e3m2_ntr<true, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2,
                                        bias, M, N, K, Y, nullptr);
  return launch_e3m2_ntr<false, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2,
                                       bias, M, N, K, Y, nullptr);
}

}  // namespace svdq
