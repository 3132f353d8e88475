// W4A4 group GEMM with the low-rank up-projection and bias fused into the epilogue.
//
// SVDQ "technical principles" / DCMP "SVDQuant": the 16-bit low-rank branch is fused into the
// low-bit kernel so it costs no extra pass over the activations.  W4A8 2.2 / 4.2: 4-bit
// weights are widened to 8 bits and fed to the INT8 units.  Per 64-group g of K the int32
// partial P[g] = qx[:, g] . qw[g, :] is exact, and
//     Y = sum_g diag(s_x[:, g]) P[g] diag(s_w[g]) + bf16(T) L2 + bias.
//
// gfx950 mapping (one workgroup = 4 waves = a 128 x 128 tile of Y; wave (wm, wn) owns the
// 64 x 64 sub-tile made of 4 x 4 tiles of 16 x 16):
//  * Staging.  Per 64-group the tile needs 128 packed rows of xq and 128 packed columns of wq
//    (32 bytes each).  Threads load 16 packed bytes per segment into registers one group ahead,
//    unpack them to int8 holding 16 * code (see unpack16_x16) and write them to LDS, so each
//    code is unpacked once per workgroup rather than once per wave.  Rows are padded to 80
//    bytes: the 16 lanes that read one MFMA fragment hit 16 disjoint bank quads.  Two LDS
//    buffers alternate, and one barrier per group separates the phases.
//  * Integer products.  v_mfma_i32_16x16x64_i8 covers exactly one group, so each result is
//    256 * P[g] for one 16 x 16 tile; operands are single 16-byte LDS reads.
//  * Scale products.  s_x[m] * s_w[n] is an outer product, which v_mfma_f32_16x16x32_f16
//    computes exactly (an fp16 x fp16 product is exact in fp32) when only k-slot 0 is nonzero:
//    lanes 0..15 keep the fp16 scale they read from LDS, lanes 16..63 zero it.
//    The dequantization is then one convert and one FMA per output and group.  The factor 256
//    of the unpacked operands is removed once, exactly, in the epilogue.
//  * W4A8 variant (A8): the activation operand arrives as 8-bit codes (W4A8 1, 2.2: 8-bit
//    activations, 4-bit weights widened onto the INT8 units).  Its 16-byte segments are only
//    reordered, with two v_perm_b32 per 8 codes, into the k order the weights' unpack gives;
//    the products then carry 16 (the weights' pre-shift) instead of 256.
//  * Epilogue.  bf16(T) [16 x 32] and L2 [32 x 16] fragments go through
//    v_mfma_f32_16x16x32_bf16 with the fp32 accumulator as C, then the bias is added and the
//    tile is rounded to bf16 (or kept fp32) and stored.
#include <type_traits>

#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

constexpr int kRowBytes = 80;  // LDS row stride of the unpacked int8 operands (64 + pad)

// Tile shape: a workgroup computes TM x TN of Y with (TM / WM) x (TN / WN) waves, each wave a
// WM x WN sub-tile of 16 x 16 MFMA fragments; PREFETCH groups of packed operands are in flight
// in registers ahead of the LDS stage being computed.
template <int TM_, int TN_, int WM_, int WN_, int PREFETCH_, int WAVES_PER_EU_>
struct GemmTile {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
  static constexpr int PREFETCH = PREFETCH_;  // groups in flight between global memory and LDS
  static constexpr int WAVES_PER_EU = WAVES_PER_EU_;  // occupancy the register budget must allow
  static_assert(PREFETCH >= 1 && PREFETCH <= 3, "prefetch depth");
  static constexpr int WAVES_N = TN / WN, WAVES = (TM / WM) * WAVES_N, THREADS = 64 * WAVES;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int kOpA = TM * kRowBytes, kOpB = TN * kRowBytes;
  static constexpr int kStageBytes = kOpA + kOpB + (TM + TN) * 2;  // A, B, s_x, s_w
  static constexpr int kLdsBytes = 2 * kStageBytes;                  // double buffer
  static_assert(2 * TM % THREADS == 0 && 2 * TN % THREADS == 0, "staging split");
  static_assert(TM + TN == THREADS || TM + TN == 2 * THREADS, "scale staging split");
};

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));

// A8: the activation operand holds 8-bit codes [M, K] (the W4A8 variant) instead of nibbles.
template <class TL, bool OUT_FP32, bool PARTIALS, int NTR, bool A8 = false>
__global__ __launch_bounds__(TL::THREADS) __attribute__((amdgpu_waves_per_eu(TL::WAVES_PER_EU)))
void w4a4_gemm_kernel(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ x_scales,
    const float* __restrict__ T, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ w_scales, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, int M, int N, int K, void* __restrict__ Y,
    int32_t* __restrict__ P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int r = 16 * NTR;
  constexpr int TM = TL::TM, TN = TL::TN, WM = TL::WM, WN = TL::WN, FM = TL::FM, FN = TL::FN;
  constexpr int kOpA = TL::kOpA, kOpB = TL::kOpB, kStageBytes = TL::kStageBytes;
  constexpr int NT = TL::THREADS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WAVES_N, wn = wave % TL::WAVES_N;
  const int rl = lane & 15, kc = lane >> 4;
  int m_tile, n_tile;  // XCD-aware order, bands of 8 row tiles
  xcd_tile_order(8, m_tile, n_tile);
  m_tile *= TM;
  n_tile *= TN;
  const int G = K / kGroup;
  const size_t ldq = (size_t)(K / 2);

  // ---- staging: segment s of an operand tile is the 16 packed bytes [16 (s & 1), +16) of row
  //      (or column) s / 2; thread t moves segments t, t + NT, ... of A and of B
  //      (8-bit activation codes: a row's group is 64 bytes, four segments of 16 codes)
  constexpr int ASEG = A8 ? 4 : 2;  // 16-byte segments per row and group
  constexpr int SA_PER = ASEG * TM / NT, SB_PER = 2 * TN / NT;
  const uint8_t* a_src[SA_PER];
  const uint8_t* b_src[SB_PER];
#pragma unroll
  for (int u = 0; u < SA_PER; ++u) {
    const int sg = tid + u * NT;
    a_src[u] = A8 ? xq + (size_t)min(m_tile + (sg >> 2), M - 1) * (size_t)K + (sg & 3) * 16
                  : xq + (size_t)min(m_tile + (sg >> 1), M - 1) * ldq + (sg & 1) * 16;
  }
#pragma unroll
  for (int u = 0; u < SB_PER; ++u) {
    const int sg = tid + u * NT;
    b_src[u] = wq + (size_t)min(n_tile + (sg >> 1), N - 1) * ldq + (sg & 1) * 16;
  }
  // scale staging: entries 0..TM-1 are s_x of the tile's rows, TM..TM+TN-1 s_w of its columns
  constexpr int SS_PER = (TM + TN) / NT;
  const uint16_t* s_src[SS_PER];
  size_t s_stride[SS_PER];
#pragma unroll
  for (int u = 0; u < SS_PER; ++u) {
    const int e = tid + u * NT;
    const bool is_a = e < TM;
    s_src[u] = PARTIALS ? nullptr
               : is_a ? x_scales + (size_t)min(m_tile + e, M - 1) * G  // s_x [M, G]
                      : w_scales + min(n_tile + e - TM, N - 1);       // s_w [G, N]
    s_stride[u] = is_a ? (size_t)1 : (size_t)N;
  }

  auto stage_ptr = [&](int buf) { return lds + buf * kStageBytes; };
  auto store_stage = [&](int buf, const v4u* a, const v4u* b, const uint16_t* sc) {
    uint8_t* st = stage_ptr(buf);
#pragma unroll
    for (int u = 0; u < SA_PER; ++u) {
      const int sg = tid + u * NT;
      if constexpr (A8) {
        // 16 codes k0..k15 in natural order -> the order unpack16_x16 gives the weights
        // (k0 k2 k4 k6 | k1 k3 k5 k7 | k8 k10 k12 k14 | k9 k11 k13 k15), so both operands of
        // the MFMA see the same k in every byte slot
        uint8_t* d = st + (sg >> 2) * kRowBytes + (sg & 3) * 16;
        const v4u v = a[u];
        *reinterpret_cast<v4u*>(d) = v4u{__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                                         __builtin_amdgcn_perm(v.y, v.x, 0x07050301u),
                                         __builtin_amdgcn_perm(v.w, v.z, 0x06040200u),
                                         __builtin_amdgcn_perm(v.w, v.z, 0x07050301u)};
      } else {
        uint8_t* d = st + (sg >> 1) * kRowBytes + (sg & 1) * 32;
        reinterpret_cast<v4i*>(d)[0] = unpack16_x16(v2u{a[u].x, a[u].y});
        reinterpret_cast<v4i*>(d)[1] = unpack16_x16(v2u{a[u].z, a[u].w});
      }
    }
#pragma unroll
    for (int u = 0; u < SB_PER; ++u) {
      const int sg = tid + u * NT;
      uint8_t* d = st + kOpA + (sg >> 1) * kRowBytes + (sg & 1) * 32;
      reinterpret_cast<v4i*>(d)[0] = unpack16_x16(v2u{b[u].x, b[u].y});
      reinterpret_cast<v4i*>(d)[1] = unpack16_x16(v2u{b[u].z, b[u].w});
    }
#pragma unroll
    for (int u = 0; u < SS_PER; ++u)
      reinterpret_cast<uint16_t*>(st + kOpA + kOpB)[tid + u * NT] = sc[u];
  };

  // ---- per-lane fragment addresses (byte offsets inside a stage)
  // A fragment i: rows wm*128 + 16 i + rl, k-chunk kc; B fragment j: columns wn*64 + 16 j + rl
  const int a_frag = (wm * WM + rl) * kRowBytes + kc * 16;
  const int b_frag = kOpA + (wn * WN + rl) * kRowBytes + kc * 16;
  // scale operands: every lane reads its row's / column's fp16 scale; only lanes 0..15 (k-slot
  // 0 of the outer-product MFMA) keep it, the others contribute zero
  const int sa_off = kOpA + kOpB + (wm * WM + rl) * 2;
  const int sb_off = kOpA + kOpB + TM * 2 + (wn * WN + rl) * 2;
  const uint32_t s_keep = kc == 0 ? 0xFFFFu : 0u;

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- global -> register prefetch ring of PD groups (slot = group % PD); LDS double buffer
  constexpr int PD = TL::PREFETCH;
  v4u ra[PD][SA_PER], rb[PD][SB_PER];
  uint16_t rs[PD][SS_PER];
  auto load_group = [&](int gg, v4u* a, v4u* b, uint16_t* sc) {
#pragma unroll
    for (int u = 0; u < SA_PER; ++u) a[u] = *reinterpret_cast<const v4u*>(a_src[u] + (size_t)gg * (A8 ? 64 : 32));
#pragma unroll
    for (int u = 0; u < SB_PER; ++u) b[u] = *reinterpret_cast<const v4u*>(b_src[u] + (size_t)gg * 32);
#pragma unroll
    for (int u = 0; u < SS_PER; ++u) sc[u] = PARTIALS ? 0 : s_src[u][(size_t)gg * s_stride[u]];
  };
#pragma unroll
  for (int k = 0; k < PD; ++k)
    if (k < G) load_group(k, ra[k], rb[k], rs[k]);
  store_stage(0, ra[0], rb[0], rs[0]);
  __syncthreads();

  // one K step: group g is in LDS buffer g & 1 and its ring slot PH is free again
  auto step = [&](int g, auto ph) {
    constexpr int PH = decltype(ph)::value, NX = (PH + 1) % PD;
    if (g + PD < G) load_group(g + PD, ra[PH], rb[PH], rs[PH]);
    const uint8_t* st = stage_ptr(g & 1);

    v4i B[FN];
    v8h_t SB[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      B[j] = *reinterpret_cast<const v4i*>(st + b_frag + j * 16 * kRowBytes);
      const uint32_t sw = *reinterpret_cast<const uint16_t*>(st + sb_off + j * 32) & s_keep;
      SB[j] = __builtin_bit_cast(v8h_t, v4u{sw, 0u, 0u, 0u});
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v4i A = *reinterpret_cast<const v4i*>(st + a_frag + i * 16 * kRowBytes);
      if constexpr (PARTIALS) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B[j], v4i{0, 0, 0, 0}, 0, 0, 0);
          const int col = n_tile + wn * WN + 16 * j + rl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = m_tile + wm * WM + 16 * i + 4 * kc + e;
            if (row < M && col < N) P[((size_t)g * M + row) * N + col] = p[e] >> (A8 ? 4 : 8);  // exact
          }
        }
      } else {
        const uint32_t sx = *reinterpret_cast<const uint16_t*>(st + sa_off + i * 32) & s_keep;
        const v8h_t SA = __builtin_bit_cast(v8h_t, v4u{sx, 0u, 0u, 0u});
        v4i p[FN];
        v4f sp[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          p[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B[j], v4i{0, 0, 0, 0}, 0, 0, 0);
          sp[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(SA, SB[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf((float)p[j][e], sp[j][e], acc[i][j][e]);
          // pin the dequantization of this fragment here: otherwise the optimizer sinks every
          // FMA below the last MFMA of the group and all MFMA results are live at once
          asm volatile("" : "+v"(acc[i][j]));
        }
      }
      // and keep the machine scheduler from hoisting the next fragment's MFMAs over this
      // fragment's dequantization
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g + 1 < G) store_stage((g + 1) & 1, ra[NX], rb[NX], rs[NX]);
    __syncthreads();
  };
  for (int g = 0; g < G; g += PD) {
    step(g, std::integral_constant<int, 0>{});
    if constexpr (PD > 1) if (g + 1 < G) step(g + 1, std::integral_constant<int, 1 % PD>{});
    if constexpr (PD > 2) if (g + 2 < G) step(g + 2, std::integral_constant<int, 2 % PD>{});
  }
  if constexpr (PARTIALS) return;

  // ---- epilogue: remove the 256 of the unpacked operands (16 with 8-bit activation codes,
  //      whose operand is not pre-shifted), low-rank up-projection, bias
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] *= A8 ? 0x1p-4f : 0x1p-8f;
  // The epilogue's addresses are loop-invariant; computed before the K loop they would stay
  // live across it and spill.  An opaque copy of the indices keeps them here.
  int row0 = m_tile + wm * WM, col0 = n_tile + wn * WN, Mo = M, No = N;
  asm volatile("" : "+v"(row0), "+v"(col0), "+s"(Mo), "+s"(No));
  if constexpr (NTR > 0) {
#pragma unroll
    for (int rk = 0; rk < (r + 31) / 32; ++rk) {
      const int kk = rk * 32 + kc * 8;  // this lane's 8 rank indices
      const bool kv = kk < r;
      v8bf Bt[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // L2p [N, r]: this lane's column, ranks kk .. kk + 7
        v4u b = v4u{0u, 0u, 0u, 0u};
        if (kv) b = *reinterpret_cast<const v4u*>(L2 + (size_t)min(col0 + 16 * j + rl, No - 1) * r + kk);
        Bt[j] = __builtin_bit_cast(v8bf, b);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        v4u a = v4u{0u, 0u, 0u, 0u};
        if (kv) {
          const v4f* tp = reinterpret_cast<const v4f*>(T + (size_t)min(row0 + 16 * i + rl, Mo - 1) * r + kk);
          const v4f t0 = tp[0], t1 = tp[1];
          a = v4u{pack2_bf16(t0.x, t0.y), pack2_bf16(t0.z, t0.w), pack2_bf16(t1.x, t1.y),
                  pack2_bf16(t1.z, t1.w)};
        }
        const v8bf At = __builtin_bit_cast(v8bf, a);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(At, Bt[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  float bj[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
    bj[j] = bias ? bf16_bits_to_float(bias[min(col0 + 16 * j + rl, No - 1)]) : 0.0f;
  if (m_tile + TM <= M && n_tile + TN <= N) {
    // a whole tile (all but the ragged edge): no per-element bounds, one uniform base and
    // fixed row offsets, and pairs of rows rounded to bf16 by one conversion (RNE); Y is
    // written once, with non-temporal stores
    const size_t base = (size_t)(m_tile + wm * WM) * N + n_tile + wn * WN;
    const uint32_t lo = (uint32_t)(4 * kc) * (uint32_t)N + (uint32_t)rl;  // < TM N
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const uint32_t o = lo + (uint32_t)(16 * i + e) * (uint32_t)N + 16 * j;
          const float v0 = acc[i][j][e] + bj[j], v1 = acc[i][j][e + 1] + bj[j];
          if constexpr (OUT_FP32) {
            float* y = reinterpret_cast<float*>(Y) + base;
            __builtin_nontemporal_store(v0, y + o);
            __builtin_nontemporal_store(v1, y + o + (uint32_t)N);
          } else {
            uint16_t* y = reinterpret_cast<uint16_t*>(Y) + base;
            const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{v0, v1}), v2bf));
            __builtin_nontemporal_store((uint16_t)w, y + o);
            __builtin_nontemporal_store((uint16_t)(w >> 16), y + o + (uint32_t)N);
          }
        }
    return;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = col0 + 16 * j + rl;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + 16 * i + 4 * kc + e;
        if (row < Mo && col < No) {
          const float v = acc[i][j][e] + bj[j];
          if constexpr (OUT_FP32)
            reinterpret_cast<float*>(Y)[(size_t)row * No + col] = v;
          else
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * No + col] = float_to_bf16_bits(v);
        }
      }
  }
}

// Tile used for every launch (see the design notes at the top of the file).  A register
// prefetch ring of one group: two groups (or the W4A8 variant's twice larger activation
// segments) spill at this occupancy and measured slower.
using Tile = GemmTile<128, 128, 64, 64, 1, 3>;

// The double-buffered stage may need more than the default 64 KB of dynamic LDS.
template <typename F>
static hipError_t allow_lds(F kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <bool OUT_FP32, bool PARTIALS, bool A8 = false>
static hipError_t launch_ntr(int ntr, dim3 grid, hipStream_t stream, const uint8_t* xq,
                             const uint16_t* x_scales, const float* T, const uint8_t* wq,
                             const uint16_t* w_scales, const uint16_t* L2, const uint16_t* bias,
                             int M, int N, int K, void* Y, int32_t* P) {
  switch (ntr) {
#define SVDQ_GEMM_CASE(n)                                                                       \
  case n: {                                                                                     \
    const hipError_t e = allow_lds(w4a4_gemm_kernel<Tile, OUT_FP32, PARTIALS, n, A8>,            \
                                   Tile::kLdsBytes);                                            \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL((w4a4_gemm_kernel<Tile, OUT_FP32, PARTIALS, n, A8>), grid,               \
                       dim3(Tile::THREADS), Tile::kLdsBytes, stream, xq, x_scales, T, wq,       \
                       w_scales, L2, bias, M, N, K, Y, P);                                      \
    break;                                                                                      \
  }
    SVDQ_GEMM_CASE(0)
    SVDQ_GEMM_CASE(1)
    SVDQ_GEMM_CASE(2)
    SVDQ_GEMM_CASE(3)
    SVDQ_GEMM_CASE(4)
    SVDQ_GEMM_CASE(5)
    SVDQ_GEMM_CASE(6)
    SVDQ_GEMM_CASE(7)
    SVDQ_GEMM_CASE(8)
#undef SVDQ_GEMM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm(const uint8_t* xq, const uint16_t* x_scales, const float* T,
                            const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                            const uint16_t* bias, int M, int N, int K, int r, void* Y,
                            int out_fp32, int32_t* partials, hipStream_t stream) {
  dim3 grid((N + Tile::TN - 1) / Tile::TN, (M + Tile::TM - 1) / Tile::TM);
  if (partials)
    return launch_ntr<false, true>(0, grid, stream, xq, nullptr, nullptr, wq, nullptr, nullptr,
                                   nullptr, M, N, K, nullptr, partials);
  if (out_fp32)
    return launch_ntr<true, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2, bias,
                                   M, N, K, Y, nullptr);
  return launch_ntr<false, false>(r / 16, grid, stream, xq, x_scales, T, wq, w_scales, L2, bias,
                                  M, N, K, Y, nullptr);
}

hipError_t launch_w4a8_gemm(const uint8_t* xq8, const uint16_t* x_scales, const float* T,
                            const uint8_t* wq, const uint16_t* w_scales, const uint16_t* L2,
                            const uint16_t* bias, int M, int N, int K, int r, void* Y,
                            int out_fp32, int32_t* partials, hipStream_t stream) {
  dim3 grid((N + Tile::TN - 1) / Tile::TN, (M + Tile::TM - 1) / Tile::TM);
  if (partials)
    return launch_ntr<false, true, true>(0, grid, stream, xq8, nullptr, nullptr, wq, nullptr,
                                         nullptr, nullptr, M, N, K, nullptr, partials);
  if (out_fp32)
    return launch_ntr<true, false, true>(r / 16, grid, stream, xq8, x_scales, T, wq, w_scales,
                                         L2, bias, M, N, K, Y, nullptr);
  return launch_ntr<false, false, true>(r / 16, grid, stream, xq8, x_scales, T, wq, w_scales, L2,
                                        bias, M, N, K, Y, nullptr);
}

}  // namespace svdq
