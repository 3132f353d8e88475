// W4A4 group GEMM on the FP6 matrix units: the INT4 codes of both operands are carried as BF6
// (E3M2) values, with the low-rank up-projection and bias fused into the epilogue.
//
// Same result as the INT8-unit GEMM (SVDQ "technical principles"; DCMP "SVDQuant" section):
//     Y = sum_g diag(s_x[:, g]) P[g] diag(s_w[g]) + bf16(T) L2 + bias,
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
//    the 32 codes k = 32 (l / 32) + i as six dwords, code i at bits 6i .. 6i+5 -- exactly slot
//    l of a (row block, group) block of the tiled container.  The 32 x 32 result: lane l holds
//    column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4, e = 0..15.
//  * Staging.  KS = 2 groups per stage, NB = 3 stages resident in LDS, two of them in flight:
//    codes and scales go from global memory straight into LDS (buffer loads with the LDS
//    destination, 16-byte and 2-byte, from a scalar buffer resource per stage), so no
//    registers or VALU work are spent on staging and the loads of stage s + 2 are issued
//    while stage s is computed.  (The epilogue's T, L2 and bias, loaded once per tile, use
//    global_load_lds.)  The tiled container's blocks are copied as they
//    are, so an MFMA operand is three ds_read_b64 per lane from its 24-byte slot.
//  * Scale products.  2 s_x[m] s_w[n] for a 32 x 32 tile is an outer product that
//    v_mfma_f32_32x32x8_f16 computes exactly (fp16 x fp16 is exact in fp32, and it is the sum
//    of two equal products) from one fp16 per lane read straight from LDS (see the operand note
//    in the kernel).  The dequantization is one FMA per output and group, so the accumulator
//    holds twice the dequantized sum -- exactly, as doubling commutes with rounding.
//  * Epilogue.  bf16(2T) [32 x 16] and L2 [16 x 32] fragments go through
//    v_mfma_f32_32x32x16_bf16 with the fp32 accumulator as C (bf16(2T) = 2 bf16(T) exactly),
//    then Y = fma(acc, 1/2, bias) is rounded to bf16 (or kept fp32) and stored: the same
//    values as without the factor 2.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

namespace f6 {
constexpr int TM = 128, TN = 128;             // workgroup tile
constexpr int KS = 2;                         // groups per stage
constexpr int NB = 3;                         // stages resident in LDS (two in flight)
constexpr int THREADS = 256;                  // 2 x 2 waves of 64 x 64
constexpr int RT = TM / 32, CT = TN / 32;     // 32 x 32 tiles along M and N
constexpr int kFrag = kE3m2Block;             // one 32-row block x one group, 64 lane slots
constexpr int kOpA = RT * KS * kFrag;         // [tile][group][64 slots][24 B]
constexpr int kOpB = CT * KS * kFrag;
constexpr int kScA = KS * TM * 4;             // [row][group], one zero-extended fp16 per dword
constexpr int kScB = KS * TN * 4;
constexpr int kStage = kScA + kScB + kOpA + kOpB;  // s_x, s_w, A, B
constexpr int kLds = NB * kStage;
constexpr int kLoadsA = kOpA / 16 / THREADS;  // 16-byte direct-to-LDS loads per thread and stage
constexpr int kLoadsB = kOpB / 16 / THREADS;
static_assert(kLoadsA * 16 * THREADS == kOpA && kLoadsB * 16 * THREADS == kOpB, "load split");
static_assert(KS * TM == THREADS && KS * TN == THREADS, "one scale per thread and operand");
static_assert(kStage % 16 == 0, "16-byte aligned stages");
}  // namespace f6

#define SVDQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// gfx9 buffer resource over [base, base + bytes): raw (stride 0), dword data format.  A load at
// an offset past `bytes` returns zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// The four resources of one stage (first group g0), all uniform (scalar registers): the codes
// of the workgroup's row and column blocks from group g0 to the end of the tensor (counted in
// 32-bit units: blocks left = (row blocks from the tile on) * G - g0 <= 2^29 for M * K <= 2^40,
// capped at 2^31 - 1 bytes, beyond every offset a stage uses); the activation scales of the
// tile's rows from group g0 on (both groups of the stage); and the TN weight scales of the
// wave's group g0 + s_gq -- or nothing when that group does not exist (the second group of an
// odd G's last stage).
struct StageRsrc {
  __amdgpu_buffer_rsrc_t a, b, sx, sw;
};
template <bool PARTIALS>
__device__ __forceinline__ StageRsrc stage_rsrc(const uint8_t* xq, const uint8_t* wq,
                                                const uint16_t* x_scales, const uint16_t* w_scales,
                                                int M, int N, int G, int mt, int nt, int m_tile,
                                                int n_tile, int g0, int s_gq, int TM, int TN) {
  constexpr int kFrag = kE3m2Block, kCap = 0x7FFFFFFF / kFrag;
  StageRsrc R;
  const int ab = ((M + 31) / 32 - mt) * G - g0, bb = ((N + 31) / 32 - nt) * G - g0;
  R.a = buffer_rsrc(xq + ((size_t)mt * G + g0) * kFrag, ab >= kCap ? 0x7FFFFFFF : ab * kFrag);
  R.b = buffer_rsrc(wq + ((size_t)nt * G + g0) * kFrag, bb >= kCap ? 0x7FFFFFFF : bb * kFrag);
  if constexpr (!PARTIALS) {
    const int g = g0 + s_gq;
    const bool live = g < G;
    // s_x is [M, G]: from the tile's first row at group g0; a lane's offset selects its row and
    // one of the stage's two groups.  The range ends after the tile's last row, so the missing
    // second group of an odd G's last stage reads nothing there (elsewhere it reads the next
    // row's first scale, which is never used)
    R.sx = buffer_rsrc(x_scales + (size_t)m_tile * G + g0, min(M - m_tile, TM) * G * 2 - 2 * g0);
    R.sw = buffer_rsrc(w_scales + (size_t)min(g, G - 1) * N + n_tile, live ? 2 * TN : 0);
  } else {
    R.sx = R.a;
    R.sw = R.b;
  }
  return R;
}

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding: vmcnt in bits 3..0
// and 15..14, expcnt 6..4, lgkmcnt 11..8)
#define SVDQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

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
  constexpr int kLoads = kLoadsA + kLoadsB + (PARTIALS ? 0 : 2);  // per thread and stage
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to SGPRs
  const int wm = wave >> 1, wn = wave & 1;
  // XCD-aware tile order in bands of 8 row tiles (of the bands 4, 8, 16 and 36 measured at
  // the FFN-up shape, 8 fetched the least from beyond L2: 246 against 418 MB per launch in
  // grid order)
  int m_tile, n_tile;
  xcd_tile_order(8, m_tile, n_tile);
  m_tile *= TM;
  n_tile *= TN;

  // ---- direct-to-LDS staging.  The codes arrive in the tiled container, whose (row block,
  //      group) blocks are exactly the MFMA operand blocks, so a stage is a copy of
  //      KS consecutive blocks per 32-row tile into LDS ([tile][group][64 slots][24 B]).  Load j
  //      of thread t moves 16-byte chunk c = j * 256 + t of the stage (each load instruction of
  //      a wave fills 1 KB of consecutive LDS, lane l at +16 l): byte 16 (c % 96) of the block
  //      (tile (c / 96) / KS, group (c / 96) % KS).  The loads are buffer loads: a uniform
  //      base (the workgroup's first row block, advanced to the stage's first group) in a buffer
  //      resource, plus a fixed 32-bit per-lane offset, so they cost no VALU work.  Each
  //      resource ends where its tensor ends, so the loads of the missing second group of an
  //      odd G's last stage read the next row block or nothing (out of range), and are never
  //      used.  Tiles past the last row block re-read that block (unused rows).
  const int G = K / kGroup;
  const int mblk = (M + 31) / 32, nblk = (N + 31) / 32;
  const int mt = m_tile / 32, nt = n_tile / 32;
  uint32_t a_off[kLoadsA], b_off[kLoadsB];  // < 4 G kFrag < 2^31 (K / 64 <= 65535)
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int c = j * THREADS + tid, blk = c / 96;
    const int tile = blk / KS;
    const size_t within = (size_t)(blk % KS) * kFrag + (c % 96) * 16;
    a_off[j] = (uint32_t)((size_t)(min(mt + tile, mblk - 1) - mt) * G * kFrag + within);
    b_off[j] = (uint32_t)((size_t)(min(nt + tile, nblk - 1) - nt) * G * kFrag + within);
  }
  // scales: thread t loads s_x of (row t / 2, group t % 2 of the stage) -- the two groups of a
  // row are adjacent in [M, G], so a wave reads 32 contiguous pairs instead of 64 scattered
  // halves (measured 2-3 % of the kernel) -- and s_w of (group t / TN, column t % TN), as
  // 2-byte direct loads, which land zero-extended in dword t of the area ([row][group] for
  // s_x, [group][column] for s_w); the group of an s_w load is uniform over the wave
  const int s_gq = wave >> 1;
  const uint32_t sx_lane =
      2u * ((uint32_t)G * (uint32_t)(min(m_tile + (tid >> 1), M - 1) - m_tile) + (uint32_t)(tid & 1));
  const uint32_t sw_lane = 2u * (uint32_t)(min(n_tile + tid % TN, N - 1) - n_tile);

  auto issue_stage = [&](int s) {
    uint8_t* st = lds + (s % NB) * kStage;
    const int g0 = s * KS;
    const StageRsrc R = stage_rsrc<PARTIALS>(xq, wq, x_scales, w_scales, M, N, G, mt, nt, m_tile,
                                             n_tile, g0, s_gq, TM, TN);
    if constexpr (!PARTIALS) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(R.sx, SVDQ_LDS(st + wave * 256), 2, sx_lane, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(R.sw, SVDQ_LDS(st + kScA + wave * 256), 2, sw_lane, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(R.a, SVDQ_LDS(st + kScA + kScB + j * 4096 + wave * 1024), 16, a_off[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(R.b, SVDQ_LDS(st + kScA + kScB + kOpA + j * 4096 + wave * 1024), 16, b_off[j], 0, 0, 0);
    }
  };

  // Load idx (0 .. kLoads - 1) of stage s alone: the main loop spreads a stage's loads over the
  // tiles of the stage before (one behind each tile's first MFMA) instead of issuing them in
  // one burst, which would hold the wave at the memory pipeline ahead of its MFMAs.
  // Order: A0, B0, A1, B1, A2, B2, then the s_x and s_w scales.
  static_assert(kLoadsA == kLoadsB && 2 * kLoadsA + 2 <= KS * 4, "one load per tile");
  auto issue_load = [&](int s, const StageRsrc& R, int idx) {
    uint8_t* st = lds + (s % NB) * kStage;
    if (idx < 2 * kLoadsA) {
      const int j = idx >> 1;
      if (idx & 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(R.b, SVDQ_LDS(st + kScA + kScB + kOpA + j * 4096 + wave * 1024), 16, b_off[j], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(R.a, SVDQ_LDS(st + kScA + kScB + j * 4096 + wave * 1024), 16, a_off[j], 0, 0, 0);
    } else if constexpr (!PARTIALS) {
      if (idx == 2 * kLoadsA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(R.sx, SVDQ_LDS(st + wave * 256), 2, sx_lane, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(R.sw, SVDQ_LDS(st + kScA + wave * 256), 2, sw_lane, 0, 0, 0);
    }
  };

  // ---- per-lane read offsets inside a stage.  MFMA operand of 32-row tile i, group gg: lane
  //      l reads its 24-byte slot at +0, +8, +16 (consecutive lanes 24 bytes apart: the 16
  //      lanes of a read phase hit 32 distinct banks).
  // One base register per 32-row tile (kept opaque): the three reads of an operand then merge
  // into one ds_read2_b64 + one ds_read_b64 that land in the operand's registers, instead of
  // being paired with the same read of the other tile.
  int a_base[2], b_base[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a_base[i] = kScA + kScB + ((2 * wm + i) * KS) * kFrag + lane * 24;
    b_base[i] = kScA + kScB + kOpA + ((2 * wn + i) * KS) * kFrag + lane * 24;
    asm volatile("" : "+v"(a_base[i]), "+v"(b_base[i]));
  }
  // scale-product operands (v_mfma_f32_32x32x8_f16): lane l supplies k-slots 4 (l / 32) .. +3
  // of row (column) l % 32.  A is (s_x[row], 0, 0, 0) -- the zero-extended dword of s_x and a
  // zero dword -- and B is (s_w[col], 0, 0, 0), in all 64 lanes, so k-slots 0 and 4 carry the
  // same exact product and the MFMA returns 2 s_x[row] s_w[col] exactly.  (Zeroing lanes
  // 32..63 instead, for s_x s_w itself, cost 8 VALU per stage in this VALU-bound loop; the
  // factor 2 is taken out exactly at the store.)
  // Rows are read pairwise swapped ((l % 32) ^ 1): element e of the scale product then belongs
  // to element e ^ 1 of the partial, so the dequantization FMA acc[e] += p[e] * s[e ^ 1] reads
  // its three operands from different VGPR banks (acc, p and s are 16-register tiles whose
  // element e would otherwise share bank e % 4, which stalls the FMA).
  const int sa_off = 2 * (32 * 2 * wm + ((lane & 31) ^ 1)) * 4;  // + (64 i + gg) * 4
  const int sb_off = kScA + (32 * 2 * wn + (lane & 31)) * 4;    // + (gg * TN + 32 j) * 4

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const v16f zero16 = acc[0][0];

  const int S = (G + KS - 1) / KS;
  issue_stage(0);
  if (S > 1) issue_stage(1);

  // ---- epilogue operands staged in LDS while the last stages run.  From iteration
  //      max(S - 2, 0) on, buffer S % NB holds no stage any more; T [128 rows x r] fp32,
  //      L2p [128 cols x r] bf16 and the bias of the tile are copied into it with the same
  //      direct-to-LDS loads, chunk-column-major (16-byte chunk c of row x at chunk index
  //      c * 128 + x) so that the epilogue's fragment reads are conflict-free.  (Without a bias
  //      the bias slot loads the weight scales instead, so every wave issues the same count.)
  constexpr bool PRE = !PARTIALS && NTR > 0 && NTR * (TM * 16 * 4 + TN * 16 * 2) + TN * 4 <= kStage;
  constexpr int kPreT = 2 * NTR, kPreL = NTR, kPre = kPreT + kPreL + 1;  // loads per thread
  constexpr int kPreL2Off = NTR * TM * 16 * 4, kPreBiasOff = kPreL2Off + NTR * TN * 16 * 2;
  auto issue_prefetch = [&]() {
    if constexpr (PRE) {
      uint8_t* pb = lds + (S % NB) * kStage;
#pragma unroll
      for (int j = 0; j < kPreT; ++j) {
        const int p = j * THREADS + tid, c = p / TM, x = p % TM;
        __builtin_amdgcn_global_load_lds(T + (size_t)min(m_tile + x, M - 1) * r + 4 * c, SVDQ_LDS(pb + j * 4096 + wave * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kPreL; ++j) {
        const int p = j * THREADS + tid, c = p / TN, x = p % TN;
        __builtin_amdgcn_global_load_lds(L2 + (size_t)min(n_tile + x, N - 1) * r + 8 * c, SVDQ_LDS(pb + kPreL2Off + j * 4096 + wave * 1024), 16, 0, 0);
      }
      const int bc = min(n_tile + (wave & 1) * 64 + lane, N - 1);
      __builtin_amdgcn_global_load_lds(bias ? bias + bc : w_scales + bc, SVDQ_LDS(pb + kPreBiasOff + (wave & 1) * 256), 2, 0, 0);
    }
  };

  // one group's MFMA operands, read from LDS
  struct Frag {
    v8i A[2], B[2];
    v4h SA[2], SB[2];
  };
  // Per-lane LDS offsets of stage s's operands, one add each per stage from an opaque stage
  // offset.  (Left to itself the compiler can turn the stage offset into an induction variable
  // with a bias that costs a second add per operand read.)
  struct Bases {
    int a[2], b[2], sa, sb;
  };
  auto bases = [&](int s) {
    int so = (s % NB) * kStage;
    asm volatile("" : "+s"(so));
    Bases Bs;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      Bs.a[i] = a_base[i] + so;
      Bs.b[i] = b_base[i] + so;
    }
    Bs.sa = sa_off + so;
    Bs.sb = sb_off + so;
    return Bs;
  };
  // operands of 32-row tile pair i (A, B, s_x, s_w of tiles i) of group gg
  auto read_half = [&](const Bases& Bs, int gg, int i, Frag& F) {
    {
      const v2u* pa = reinterpret_cast<const v2u*>(lds + Bs.a[i] + gg * kFrag);
      const v2u* pb = reinterpret_cast<const v2u*>(lds + Bs.b[i] + gg * kFrag);
      const v2u a0 = pa[0], a1 = pa[1], a2 = pa[2];
      const v2u b0 = pb[0], b1 = pb[1], b2 = pb[2];
      F.A[i] = v8i{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
      F.B[i] = v8i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y, (int)b2.x, (int)b2.y, 0, 0};
      if constexpr (!PARTIALS) {
        const uint32_t sx = *reinterpret_cast<const uint32_t*>(lds + Bs.sa + (64 * i + gg) * 4);
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(lds + Bs.sb + (gg * TN + 32 * i) * 4);
        F.SA[i] = __builtin_bit_cast(v4h, v2u{sx, 0u});
        F.SB[i] = __builtin_bit_cast(v4h, v2u{sw, 0u});
      }
    }
  };
  auto read_frag = [&](const Bases& Bs, int gg, Frag& F) {
    read_half(Bs, gg, 0, F);
    read_half(Bs, gg, 1, F);
  };
  auto fma8 = [](v16f& a, const v16f& p, const v16f& sp, int half) {
#pragma unroll
    for (int e = 8 * half; e < 8 * half + 8; ++e) a[e] = __builtin_fmaf(p[e], sp[e ^ 1], a[e]);
  };
  // stage s is complete in LDS for every wave: own loads drained down to the next stage's,
  // then a barrier (which also frees stage s - 1's buffer for stage s + 2)
  //  (a bare s_barrier: __syncthreads() would add a fence that drains every load in flight,
  //  including the next stage's)
  auto wait_stage = [&](int s) {
    if (s + 1 < S)
      SVDQ_WAIT_VMCNT(kLoads);
    else if (PRE && S >= 2)  // the epilogue's prefetch, issued a stage earlier, may stay in flight
      SVDQ_WAIT_VMCNT(kPre);
    else
      SVDQ_WAIT_VMCNT(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if constexpr (PARTIALS) {
    for (int s = 0; s < S; ++s) {
      wait_stage(s);
      if (s + 2 < S) issue_stage(s + 2);
      const Bases Bs = bases(s);
      const int ng = min(KS, G - s * KS);
      for (int gg = 0; gg < ng; ++gg) {
        Frag F;
        read_frag(Bs, gg, F);
        const int g = s * KS + gg;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.A[i], F.B[j], zero16, 3, 3, 0, 127, 0, 127);
            const int col = n_tile + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = m_tile + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              if (row < M && col < N) P[((size_t)g * M + row) * N + col] = (int32_t)p[e];  // exact
            }
          }
      }
    }
    return;
  } else {
    // Software pipeline with a lag of one 32 x 32 tile: the 16 FMAs that dequantize tile t are
    // issued in two halves behind the two MFMAs of tile t + 1, so the VALU works while the
    // matrix unit does.  The last tile of a stage, (1, 1), is dequantized at the start of the
    // next stage, under the LDS reads of that stage's first operands.
    v16f pp = zero16, spp = zero16;  // partial and scale product of the pending tile (1, 1)
    // one stage; ISSUE: the loads of stage s + 2 are issued one per tile (every stage but the
    // last two)
    auto stage = [&](int s, auto issue_tag) {
      constexpr bool ISSUE = decltype(issue_tag)::value;
      StageRsrc R2{};
      if constexpr (ISSUE)
        R2 = stage_rsrc<false>(xq, wq, x_scales, w_scales, M, N, G, mt, nt, m_tile, n_tile,
                               (s + 2) * KS, s_gq, TM, TN);
      wait_stage(s);
      if (s == max(S - 2, 0)) issue_prefetch();
      const Bases Bs = bases(s);
      const int ng = min(KS, G - s * KS);
      Frag F[KS];
      read_frag(Bs, 0, F[0]);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[1][1][e] = __builtin_fmaf(pp[e], spp[e ^ 1], acc[1][1][e]);
      asm volatile("" : "+v"(acc[1][1]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gg = 0; gg < KS; ++gg) {
        if (gg >= ng) break;  // uniform (only in the last stage, which issues nothing)
        const Frag& C = F[gg];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int i = t >> 1, j = t & 1, li = gg * 4 + t;
          const v16f sn = __builtin_amdgcn_mfma_f32_32x32x8f16(C.SA[i], C.SB[j], zero16, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (ISSUE && li < kLoads) issue_load(s + 2, R2, li);
          // (also in a last stage without a second group: its LDS holds a valid duplicate)
          if (t < 2 && gg + 1 < KS) read_half(Bs, gg + 1, t, F[gg + 1]);
          // the pending tile: (1, 1) of the previous group at t == 0, else tile t - 1
          const int pi = t == 0 ? 1 : (t - 1) >> 1, pj = t == 0 ? 1 : (t - 1) & 1;
          const bool have = t > 0 || gg > 0;
          if (have) fma8(acc[pi][pj], pp, spp, 0);
          const v16f pn = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(C.A[i], C.B[j], zero16, 3, 3, 0, 127, 0, 127);
          if (have) {
            fma8(acc[pi][pj], pp, spp, 1);
            asm volatile("" : "+v"(acc[pi][pj]));
          }
          pp = pn;
          spp = sn;
          // issue order: MFMA (scale product of tile t, the longer-latency one, so its result
          // is ready when the next tile's first FMAs read it), the stage load, 8 VALU (first
          // half of the pending tile), MFMA (partial of tile t), 8 VALU -- the pending tile's
          // registers stay distinct from tile t's, and each MFMA runs under the work behind it
          // (the scale product first measured 1 % faster than the partial first)
          if (ISSUE && li < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          if (t < 2 && gg + 1 < KS)  // the next group's operand reads go under this MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    int s = 0;
    for (; s + 2 < S; ++s) stage(s, BoolTag<true>{});
    for (; s < S; ++s) stage(s, BoolTag<false>{});
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[1][1][e] = __builtin_fmaf(pp[e], spp[e ^ 1], acc[1][1][e]);
  }

  // ---- epilogue: low-rank up-projection, bias, store.  The addresses are loop-invariant;
  //      computed before the K loop they would stay live across it, so they go through an
  //      opaque copy here.
  int row0 = m_tile + wm * 64, col0 = n_tile + wn * 64, Mo = M, No = N;
  asm volatile("" : "+v"(row0), "+v"(col0), "+s"(Mo), "+s"(No));
  const int l32 = lane & 31, hi = lane >> 5;
  const uint8_t* pb = lds + (S % NB) * kStage;
  if constexpr (PRE) {  // the staged T, L2 and bias are complete for every wave
    SVDQ_WAIT_VMCNT(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if constexpr (PRE) {
#pragma unroll
    for (int kk = 0; kk < r; kk += 16) {
      const int k8 = kk + 8 * hi;  // this lane's 8 rank indices: T chunks k8 / 4 and + 1
      v8bf Bt[2], At[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)  // L2p: this lane's column, ranks k8 .. k8 + 7
        Bt[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(pb + kPreL2Off + ((k8 / 8) * TN + wn * 64 + 32 * j + l32) * 16));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int x = wm * 64 + 32 * i + l32;
        const v4f t0 = *reinterpret_cast<const v4f*>(pb + ((k8 / 4) * TM + x) * 16);
        const v4f t1 = *reinterpret_cast<const v4f*>(pb + ((k8 / 4 + 1) * TM + x) * 16);
        const float tv[8] = {2.0f * t0.x, 2.0f * t0.y, 2.0f * t0.z, 2.0f * t0.w,
                             2.0f * t1.x, 2.0f * t1.y, 2.0f * t1.z, 2.0f * t1.w};  // exact
        At[i] = to_bf16x8(tv);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[i], Bt[j], acc[i][j], 0, 0, 0);
    }
  } else if constexpr (NTR > 0) {
#pragma unroll
    for (int kk = 0; kk < r; kk += 16) {
      const int k8 = kk + 8 * hi;  // this lane's 8 rank indices
      v8bf Bt[2], At[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)  // L2p: this lane's column, ranks k8 .. k8 + 7
        Bt[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(L2 + (size_t)min(col0 + 32 * j + l32, No - 1) * r + k8));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4f* tp = reinterpret_cast<const v4f*>(T + (size_t)min(row0 + 32 * i + l32, Mo - 1) * r + k8);
        const v4f t0 = tp[0], t1 = tp[1];
        const float tv[8] = {2.0f * t0.x, 2.0f * t0.y, 2.0f * t0.z, 2.0f * t0.w,
                             2.0f * t1.x, 2.0f * t1.y, 2.0f * t1.z, 2.0f * t1.w};  // exact
        At[i] = to_bf16x8(tv);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[i], Bt[j], acc[i][j], 0, 0, 0);
    }
  }
  float bj[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (bias) {
      if constexpr (PRE)
        bj[j] = bf16_bits_to_float((uint16_t)*reinterpret_cast<const uint32_t*>(pb + kPreBiasOff + (wn * 64 + 32 * j + l32) * 4));
      else
        bj[j] = bf16_bits_to_float(bias[min(col0 + 32 * j + l32, No - 1)]);
    }
  }
  if (m_tile + TM <= M && n_tile + TN <= N) {
    // a whole tile (all but the ragged edge): no per-element bounds, one uniform base and
    // fixed row offsets, and pairs of rows rounded to bf16 by one conversion (RNE).  Y is
    // written once and not read here: non-temporal stores stream it out instead of leaving it
    // dirty in the caches, where the next kernel's reads would wait on its write-back (the
    // activation pass of the next step: 26.5 -> 22.6 us).
    const size_t base = (size_t)(m_tile + wm * 64) * N + n_tile + wn * 64;
    const uint32_t lo = (uint32_t)(4 * hi) * (uint32_t)N + (uint32_t)l32;  // < 128 N
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {  // rows e and e + 1 are consecutive (e % 4 in {0, 2})
          const uint32_t o = lo + (uint32_t)(32 * i + 8 * (e >> 2) + (e & 3)) * (uint32_t)N + 32 * j;
          const float v0 = __builtin_fmaf(acc[i][j][e], 0.5f, bj[j]);
          const float v1 = __builtin_fmaf(acc[i][j][e + 1], 0.5f, bj[j]);
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
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + 32 * j + l32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < Mo && col < No) {
          const float v = __builtin_fmaf(acc[i][j][e], 0.5f, bj[j]);
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
  case n: {                                                                                    \
    /* the three resident stages need more than the default 64 KB of dynamic LDS */            \
    const hipError_t e = hipFuncSetAttribute(                                                  \
        reinterpret_cast<const void*>(w4a4_gemm_e3m2_kernel<OUT_FP32, PARTIALS, n>),            \
        hipFuncAttributeMaxDynamicSharedMemorySize, f6::kLds);                                 \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((w4a4_gemm_e3m2_kernel<OUT_FP32, PARTIALS, n>), grid, dim3(f6::THREADS), \
                       f6::kLds, stream, xq, x_scales, T, wq, w_scales, L2, bias, M, N, K, Y,   \
                       P);                                                                     \
    break;                                                                                     \
  }
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
