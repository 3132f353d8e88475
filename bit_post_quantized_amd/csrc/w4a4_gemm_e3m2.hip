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
// gfx950 mapping.  One workgroup = 8 waves = a 256 x 128 tile of Y, one workgroup per CU.
// The waves form four positions of 128 x 64 (2 x 2) and two k-halves: the waves of a position
// share its outputs and split the groups, wave (p, h) taking group 2 s + h of stage s, and the
// two halves' sums meet in LDS at the end.  Each SIMD thus runs two waves (one per half), whose
// matrix and vector work interleave, while each wave's 4 x 2 tiles of 32 x 32 read every
// operand from LDS once per two (A) or four (B) products: on this chip the operand reads out
// of LDS, not the matrix or vector units, bound a GEMM with per-group dequantization.
//  * MFMA operand layout (32 x 32 x 64 f8f6f4, BF6): lane l supplies row (or column) l % 32 and
//    the 32 codes k = 32 (l / 32) + i as six dwords, code i at bits 6i .. 6i+5 -- exactly slot
//    l of a (row block, group) block of the tiled container.  The 32 x 32 result: lane l holds
//    column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4, e = 0..15.
//  * Staging.  A stage holds two groups (one per k-half); four stages are resident in LDS.
//    Codes and scales go from global memory straight into LDS (buffer loads with the LDS
//    destination, 16-byte codes and 2-byte scales), six loads per wave and stage, issued two
//    stages ahead over the second half of a stage.  One barrier per stage, in its middle: it
//    publishes the next stage and frees the buffer of the stage before the current one.  The
//    tiled container's blocks are copied as they are, so an operand is three ds_read_b64 per
//    lane from its 24-byte slot.
//  * Scale products.  s_x[m] * s_w[n] for a 32 x 32 tile is an outer product that
//    v_mfma_f32_32x32x8_f16 computes exactly (fp16 x fp16 is exact in fp32) from one fp16 per
//    lane read from LDS, with every k-slot but one zero.  The dequantization is one FMA per
//    output and group, one tile behind the MFMAs.
//  * Epilogue.  The low-rank product bf16(T) [32 x 16] x L2 [16 x 32] runs on
//    v_mfma_f32_32x32x16_bf16 with the fp32 accumulator as C (rank chunks split between the
//    halves), T, L2 and the bias having been staged in LDS during the last stages; then each
//    half finalizes one 64-column half of the position's outputs, adding the other half's sums
//    from LDS, the bias, rounding to bf16 (or keeping fp32) and storing.
//  * Tile order.  Workgroup b runs on XCD b mod 8.  When the column tiles split evenly, each XCD
//    owns a strip of column tiles and walks the row tiles inside it, so the weight panels of
//    its strip stay in its L2 and the activation panel of a row tile is read by the strip's
//    workgroups together.
#include "svdq_device.hpp"
#include "svdq_launch.hpp"

namespace svdq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

namespace f6 {
constexpr int TM = 256, TN = 128;             // workgroup tile
constexpr int KS = 2;                         // groups per stage (one per k-half)
constexpr int NB = 4;                         // stage buffers in LDS
constexpr int THREADS = 512;                  // 4 positions x 2 k-halves
constexpr int kFrag = kE3m2Block;             // one 32-row block x one group, 64 lane slots
constexpr int kRT = TM / 32, kCT = TN / 32;   // 32-row blocks of the tile (8, 4)
constexpr int kOpA = kRT * KS * kFrag;        // [row block][group][64 slots][24 B]
constexpr int kOpB = kCT * KS * kFrag;
constexpr int kScA = KS * TM * 4;             // [group][row], one zero-extended fp16 per dword
constexpr int kScB = KS * TN * 4;
constexpr int kOffB = kOpA, kOffSx = kOpA + kOpB, kOffSw = kOffSx + kScA;
constexpr int kStage = kOpA + kOpB + kScA + kScB;
constexpr int kLds = NB * kStage;
constexpr int kLoads = 6;                     // direct-to-LDS loads per wave and stage
static_assert(kOpA == 3 * THREADS * 16 && kOpB == 3 * (THREADS / 2) * 16, "load split");
static_assert(kStage % 16 == 0 && kLds <= 160 * 1024, "LDS budget");
// exchange of the k-halves' sums: [wave][tile i][e / 4][lane][4 floats]
static_assert(8 * 4 * 4 * 64 * 16 <= kLds, "exchange area");
}  // namespace f6

#define SVDQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// gfx9 buffer resource over [base, base + bytes): raw (stride 0), dword data format.  A load at
// an offset past `bytes` returns zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding: vmcnt in bits 3..0
// and 15..14, expcnt 6..4, lgkmcnt 11..8)
#define SVDQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ int cap_bytes(long long b) {
  return b <= 0 ? 0 : b >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)b;
}

__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Output tile of workgroup b: (row tile, column tile).
__device__ __forceinline__ void tile_of(int b, int mtiles, int ntiles, int& mi, int& ni) {
  const int total = mtiles * ntiles;
  if (ntiles % 8 == 0 && total % 8 == 0) {
    // XCD x = b % 8 walks, in order, the row tiles of its strip of ntiles / 8 column tiles
    const int per = total / 8, w = ntiles / 8;
    const int k = (b & 7) * per + (b >> 3);
    const int strip = k / per, kk = k % per;
    mi = kk / w;
    ni = strip * w + kk % w;
  } else {
    mi = b / ntiles;
    ni = b % ntiles;
  }
}

template <bool OUT_FP32, bool PARTIALS, int NTR>
__global__ __launch_bounds__(f6::THREADS) void w4a4_gemm_e3m2_kernel(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ x_scales,
    const float* __restrict__ T, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ w_scales, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, int M, int N, int K, void* __restrict__ Y,
    int32_t* __restrict__ P) {
  using namespace f6;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int r = 16 * NTR;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to SGPRs
  const int h = wave >> 2, pos = wave & 3, wm = pos >> 1, wn = pos & 1;
  const int G = K / kGroup;
  const int mblk = (M + 31) / 32, nblk = (N + 31) / 32;
  int mi, ni;
  tile_of(blockIdx.x, (M + TM - 1) / TM, (N + TN - 1) / TN, mi, ni);
  const int m_tile = mi * TM, n_tile = ni * TN;
  const int mt = m_tile / 32, nt = n_tile / 32;
  const int S = (G + KS - 1) / KS;

  // ---- direct-to-LDS staging: per stage s (groups g0 = 2 s, g0 + 1), each wave issues six
  //      loads.  Codes: 16-byte chunk c of the stage's A area ([row block][group][1536 B]) is
  //      A load j of thread t with c = 512 j + t (every wave instruction fills 1 KB of
  //      consecutive LDS, lane l at +16 l); B chunks likewise, 2 loads for waves 0..3 and 1
  //      for waves 4..7.  Scales: wave w loads s_x of group w / 4 for 64 rows; waves 4..7 load
  //      s_w of group (w - 4) / 2 for 64 columns; a 2-byte load lands zero-extended in the
  //      lane's dword.  The code loads are buffer loads from a uniform base (the tile's first
  //      row block at group g0) plus a fixed per-lane offset; rows past the last row block
  //      re-read that block (unused).
  uint32_t a_off[3], b_off[2];  // < 9 G kFrag < 2^31 (K / 64 <= 65535)
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = j * THREADS + tid, blk = c / 96;
    a_off[j] = (uint32_t)((size_t)(min(mt + (blk >> 1), mblk - 1) - mt) * G * kFrag +
                          (size_t)(blk & 1) * kFrag + (c % 96) * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wave < 4 ? j * 256 + tid : 512 + (tid - 256), blk = c / 96;
    b_off[j] = (uint32_t)((size_t)(min(nt + (blk >> 1), nblk - 1) - nt) * G * kFrag +
                          (size_t)(blk & 1) * kFrag + (c % 96) * 16);
  }
  // scale loads: s_x is [M, G] (row-major): this lane's row, the group advances by 2 bytes
  const int sx_g = wave >> 2;
  const int sx_row = min(m_tile + 64 * (wave & 3) + lane, M - 1);
  const uint32_t sx_lane = (uint32_t)(sx_row - m_tile) * (uint32_t)G * 2u;  // < 256 G 2
  const int sw_g = (wave - 4) >> 1;  // waves 4..7
  const uint32_t sw_lane = 2u * (uint32_t)(min(n_tile + 64 * ((wave - 4) & 1) + lane, N - 1) - n_tile);
  // code blocks from the tile's first row (column) block to the tensor's end (<= 2^29), and the
  // byte range of a resource that starts at group g0 (capped at 2^31 - 1, far beyond every
  // offset a stage uses)
  constexpr int kCapBlocks = 0x7FFFFFFF / kFrag;
  const int a_blocks = (mblk - mt) * G, b_blocks = (nblk - nt) * G;
  const int sx_bytes = min(M - m_tile, TM) * G * 2;  // the tile's rows of s_x from group 0
  auto blocks_bytes = [](int blocks) { return blocks >= kCapBlocks ? 0x7FFFFFFF : blocks * kFrag; };

  // scale resources (uniform per wave and stage); a group past the last gives an empty range
  auto sx_rsrc = [&](int g) {
    if (PARTIALS || g >= G) return buffer_rsrc(xq, 0);
    return buffer_rsrc(x_scales + (size_t)m_tile * G + g, sx_bytes - 2 * g);
  };
  auto sw_rsrc = [&](int g) {
    if (PARTIALS || g >= G) return buffer_rsrc(wq, 0);
    return buffer_rsrc(w_scales + (size_t)g * N + n_tile, 2 * min(TN, N - n_tile));
  };

  // Load idx (0 .. 5) of stage s.  Waves 0..3: A0 B0 A1 B1 A2 s_x; waves 4..7: A0 B0 A1 s_w A2
  // s_x.
  auto issue_load = [&](int s, int idx) {
    uint8_t* st = lds + (s % NB) * kStage;
    const int g0 = s * KS;
    if (idx == 0 || idx == 2 || idx == 4) {
      const int j = idx >> 1;
      const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(xq + ((size_t)mt * G + g0) * kFrag, blocks_bytes(a_blocks - g0));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, SVDQ_LDS(st + j * 8192 + wave * 1024), 16, a_off[j], 0, 0, 0);
    } else if (idx == 1 || (idx == 3 && wave < 4)) {
      const int j = idx >> 1;
      const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(wq + ((size_t)nt * G + g0) * kFrag, blocks_bytes(b_blocks - g0));
      uint8_t* dst = wave < 4 ? st + kOffB + j * 4096 + wave * 1024 : st + kOffB + 8192 + (wave - 4) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, SVDQ_LDS(dst), 16, b_off[j], 0, 0, 0);
    } else if (idx == 3) {  // waves 4..7: s_w (the partials load nothing, same count)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sw_rsrc(g0 + sw_g), SVDQ_LDS(st + kOffSw + sw_g * 512 + ((wave - 4) & 1) * 256), 2, sw_lane, 0, 0, 0);
    } else {  // idx == 5: s_x
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sx_rsrc(g0 + sx_g), SVDQ_LDS(st + kOffSx + sx_g * 1024 + (wave & 3) * 256), 2, sx_lane, 0, 0, 0);
    }
  };
  auto issue_stage = [&](int s) {
#pragma unroll
    for (int idx = 0; idx < kLoads; ++idx) issue_load(s, idx);
  };

  // ---- epilogue operands (T [256 rows x r] fp32, L2 [r x 128 columns] bf16, bias [128]),
  //      staged in the two buffers that are free from the barrier that publishes the last
  //      stage on: T chunk-column-major (16-byte chunk c of row x at chunk c * 256 + x), L2 and
  //      the bias as zero-extended dwords ([rank][column], then the bias).
  constexpr bool PRE = !PARTIALS && NTR > 0 && NTR <= 2;
  constexpr int kPreT = 2 * NTR, kPreL = 4 * NTR;  // loads per thread
  // (issued once, late in the loop: the lane index goes through an opaque copy so that none of
  //  these addresses is computed early and held across the loop)
  auto issue_prefetch = [&]() {
    if constexpr (PRE) {
      uint8_t* bt = lds + (S % NB) * kStage;
      uint8_t* bl = lds + ((S + 1) % NB) * kStage;
      int t_ = tid;
      asm volatile("" : "+v"(t_));
      // T rows: chunk p = 512 j + t covers row p % 256, floats 4 (p / 256) .. +3
      const __amdgpu_buffer_rsrc_t rt = buffer_rsrc(T + (size_t)m_tile * r, min(M - m_tile, TM) * r * 4);
      const uint32_t trow = (uint32_t)(t_ & (TM - 1)) * (uint32_t)(r * 4);
#pragma unroll
      for (int j = 0; j < kPreT; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, SVDQ_LDS(bt + j * 8192 + wave * 1024), 16, trow + 16u * (uint32_t)((j * THREADS + t_) / TM), 0, 0, 0);
      // L2 [r, N]: element p = 512 j + t is rank p / 128, column p % 128 (clamped to N - 1)
      const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(L2 + n_tile, cap_bytes((long long)(r - 1) * N * 2 + 2LL * (N - n_tile)));
      const uint32_t lcol = 2u * (uint32_t)(min(n_tile + (t_ & (TN - 1)), N - 1) - n_tile);
#pragma unroll
      for (int j = 0; j < kPreL; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, SVDQ_LDS(bl + j * 2048 + wave * 256), 2, lcol + (uint32_t)((j * THREADS + t_) / TN) * (uint32_t)N * 2u, 0, 0, 0);
      if (bias && wave < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(bias + n_tile, 2 * min(TN, N - n_tile)), SVDQ_LDS(bl + r * TN * 4 + wave * 256), 2, lcol, 0, 0, 0);
    }
  };

  // ---- LDS read offsets inside a stage (this wave's group: h): a uniform part per operand
  //      kind plus one per-lane term each; tile i (j) adds a constant.
  const uint32_t lane24 = (uint32_t)lane * 24;
  const int a_wave = (8 * wm + h) * kFrag;            // + 2 i kFrag for row block 4 wm + i
  const int b_wave = kOffB + (4 * wn + h) * kFrag;    // + 2 j kFrag
  // scale-product operands (v_mfma_f32_32x32x8_f16): lane l supplies k-slots 4 (l / 32) .. +3
  // of row (column) l % 32.  A is (s_x[row], 0, 0, 0) and B is (s_w[col], 0, 0, 0) in lanes
  // 0..31 and zero in lanes 32..63, so only k-slot 0 contributes and the MFMA returns
  // s_x[row] * s_w[col] exactly.  Rows are read pairwise swapped ((l % 32) ^ 1): element e of
  // the scale product then belongs to element e ^ 1 of the partial, so the dequantization FMA
  // acc[e] += p[e] * s[e ^ 1] reads its three operands from different VGPR banks.
  const int sa_wave = kOffSx + h * (TM * 4) + 512 * wm;  // + 128 i
  const int sb_wave = kOffSw + h * (TN * 4) + 256 * wn;  // + 128 j
  const uint32_t sa_lane = 4u * (uint32_t)((lane & 31) ^ 1), sb_lane = 4u * (uint32_t)(lane & 31);
  const uint32_t keep = lane < 32 ? 0xFFFFFFFFu : 0u;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const v16f zero16 = acc[0][0];

  auto read_op = [&](const uint8_t* p) -> v8i {
    const v2u* q = reinterpret_cast<const v2u*>(p);
    const v2u a0 = q[0], a1 = q[1], a2 = q[2];
    return v8i{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
  };
  auto read_a = [&](const uint8_t* st, int i) { return read_op(st + a_wave + lane24 + 2 * i * kFrag); };
  auto read_b = [&](const uint8_t* st, int j) { return read_op(st + b_wave + lane24 + 2 * j * kFrag); };
  auto read_sa = [&](const uint8_t* st, int i) -> v4h {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(st + sa_wave + sa_lane + 128 * i);
    return __builtin_bit_cast(v4h, v2u{v & keep, 0u});
  };
  auto read_sb = [&](const uint8_t* st, int j) -> v4h {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(st + sb_wave + sb_lane + 128 * j);
    return __builtin_bit_cast(v4h, v2u{v & keep, 0u});
  };

  // ---- prologue: stages 0 and 1 in flight, wait for stage 0, publish it, then stage 2
  issue_stage(0);
  if (S > 1) issue_stage(1);
  if (S > 1)
    SVDQ_WAIT_VMCNT(kLoads);
  else
    SVDQ_WAIT_VMCNT(0);
  stage_barrier();
  if (S > 2) issue_stage(2);
  if (S == 1) issue_prefetch();

  if constexpr (PARTIALS) {
    for (int s = 0; s < S; ++s) {
      if (s > 0) {  // stage s published (its loads done), buffer of stage s - 2 free
        if (s + 1 < S)
          SVDQ_WAIT_VMCNT(kLoads);
        else
          SVDQ_WAIT_VMCNT(0);
        stage_barrier();
        if (s + 2 < S) issue_stage(s + 2);
      }
      const uint8_t* st = lds + (s % NB) * kStage;
      const int g = s * KS + h;
      if (g < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(read_a(st, i), read_b(st, j), zero16, 3, 3, 0, 127, 0, 127);
            const int col = n_tile + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = m_tile + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              if (row < M && col < N) P[((size_t)g * M + row) * N + col] = (int32_t)p[e];  // exact
            }
          }
      }
    }
    return;
  } else {
    // Operands: B[0], B[1] for the whole stage, A in a ring of two (A[i] is read two tiles
    // ahead), the scale operands one tile ahead.  The next stage's first operands are read in
    // the last two tiles, after the barrier that publishes them.  A group that does not exist
    // (the second of an odd G's last stage) computes from whatever its LDS slots hold (every
    // BF6 pattern is finite) with zero scales, adding zero.
    v8i Bop[2], Aop[2];
    v4h SA[2], SB[2];
    Bop[0] = read_b(lds, 0);
    Bop[1] = read_b(lds, 1);
    Aop[0] = read_a(lds, 0);
    SA[0] = read_sa(lds, 0);
    SB[0] = read_sb(lds, 0);
    SB[1] = read_sb(lds, 1);
    // partial and scale product of tile t in slot t % 2; the FMAs of tile t - 1 read the other
    v16f Pb[2], Sb[2];
    Pb[1] = zero16;
    Sb[1] = zero16;

    for (int s = 0; s < S; ++s) {
      const uint8_t* st = lds + (s % NB) * kStage;
      const uint8_t* sn_st = lds + ((s + 1) % NB) * kStage;
      const bool more = s + 1 < S;          // a next stage exists
      const bool load3 = s + 3 < S;         // its loads are issued in this stage's second half
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = t >> 1, j = t & 1, cur = t & 1, prv = cur ^ 1;
        if (t == 4 && more) {
          // stage s + 1 complete for every wave; stage s - 1 finished by every wave
          if (s + 2 < S)
            SVDQ_WAIT_VMCNT(kLoads);
          else
            SVDQ_WAIT_VMCNT(0);
          stage_barrier();
          if (s + 2 == S) issue_prefetch();
        }
        Sb[cur] = __builtin_amdgcn_mfma_f32_32x32x8f16(SA[i & 1], SB[j], zero16, 0, 0, 0);
        // stage loads of s + 3 (into the buffer of s - 1): two, two, one, one over tiles 4..7
        if (t >= 4 && load3) {
          if (t == 4) {
            issue_load(s + 3, 0);
            issue_load(s + 3, 1);
          } else if (t == 5) {
            issue_load(s + 3, 2);
            issue_load(s + 3, 3);
          } else {
            issue_load(s + 3, t - 2);
          }
        }
        // operand reads ahead
        if (t == 0 || t == 2 || t == 4) Aop[(i + 1) & 1] = read_a(st, i + 1);
        if (t == 1 || t == 3 || t == 5) SA[((t + 1) >> 1) & 1] = read_sa(st, (t + 1) >> 1);
        // the pending tile: (3, 1) of the previous stage at t == 0, else tile t - 1
        const int pi = t == 0 ? 3 : (t - 1) >> 1, pj = t == 0 ? 1 : (t - 1) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[pi][pj][e] = __builtin_fmaf(Pb[prv][e], Sb[prv][e ^ 1], acc[pi][pj][e]);
        Pb[cur] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Aop[i & 1], Bop[j], zero16, 3, 3, 0, 127, 0, 127);
#pragma unroll
        for (int e = 8; e < 16; ++e) acc[pi][pj][e] = __builtin_fmaf(Pb[prv][e], Sb[prv][e ^ 1], acc[pi][pj][e]);
        asm volatile("" : "+v"(acc[pi][pj]));
        // next stage's first operands (published by the barrier at tile 4)
        if (t == 6) {
          Bop[0] = read_b(sn_st, 0);
          Aop[0] = read_a(sn_st, 0);
          SB[0] = read_sb(sn_st, 0);
        }
        if (t == 7) {
          Bop[1] = read_b(sn_st, 1);
          SB[1] = read_sb(sn_st, 1);
          SA[0] = read_sa(sn_st, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[3][1][e] = __builtin_fmaf(Pb[1][e], Sb[1][e ^ 1], acc[3][1][e]);
  }

  // ---- epilogue.  Every wave's loads (the staged T, L2, bias) complete, every wave done with
  //      the stage buffers.
  SVDQ_WAIT_VMCNT(0);
  stage_barrier();
  int row0 = m_tile + wm * 128, col0 = n_tile + wn * 64, Mo = M, No = N;
  asm volatile("" : "+v"(row0), "+v"(col0), "+s"(Mo), "+s"(No));
  const int l32 = lane & 31, hi = lane >> 5;
  // low-rank up-projection: rank chunk c (16 ranks) on k-half c % 2
  if constexpr (NTR > 0) {
    const uint8_t* bt = lds + (S % NB) * kStage;
    const uint8_t* bl = lds + ((S + 1) % NB) * kStage;
#pragma unroll
    for (int c = 0; c < NTR; ++c) {
      if ((c & 1) != h) continue;
      const int k8 = 16 * c + 8 * hi;  // this lane's 8 rank indices
      v8bf Bt[2], At[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint16_t b;
          if constexpr (PRE)
            b = (uint16_t)*reinterpret_cast<const uint32_t*>(bl + ((k8 + q) * TN + wn * 64 + 32 * j + l32) * 4);
          else
            b = L2[(size_t)(k8 + q) * No + min(col0 + 32 * j + l32, No - 1)];
          v[q] = bf16_bits_to_float(b);
        }
        Bt[j] = to_bf16x8(v);  // exact: bf16 values
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4f t0, t1;
        if constexpr (PRE) {
          const int x = wm * 128 + 32 * i + l32;
          t0 = *reinterpret_cast<const v4f*>(bt + ((k8 / 4) * TM + x) * 16);
          t1 = *reinterpret_cast<const v4f*>(bt + ((k8 / 4 + 1) * TM + x) * 16);
        } else {
          const v4f* tp = reinterpret_cast<const v4f*>(T + (size_t)min(row0 + 32 * i + l32, Mo - 1) * r + k8);
          t0 = tp[0];
          t1 = tp[1];
        }
        const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
        At[i] = to_bf16x8(tv);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[i], Bt[j], acc[i][j], 0, 0, 0);
    }
  }
  // this half finalizes column tile j = h of the position
  float bj = 0.0f;
  if (bias) {
    if constexpr (PRE)
      bj = bf16_bits_to_float((uint16_t)*reinterpret_cast<const uint32_t*>(lds + ((S + 1) % NB) * kStage + r * TN * 4 + (wn * 64 + 32 * h + l32) * 4));
    else
      bj = bf16_bits_to_float(bias[min(col0 + 32 * h + l32, No - 1)]);
  }
  stage_barrier();  // the staged epilogue operands are read
  // exchange: wave (pos, h) sends its sums of column tile 1 - h to wave (pos, 1 - h), and
  // finalizes column tile h: its own sums + the partner's + the bias
  auto send = [&](const v16f (&a)[4]) {
    uint8_t* out = lds + ((size_t)(pos * 2 + (1 - h)) * 4) * 4 * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<v4f*>(out + ((i * 4 + e4) * 64 + lane) * 16) =
            v4f{a[i][4 * e4], a[i][4 * e4 + 1], a[i][4 * e4 + 2], a[i][4 * e4 + 3]};
  };
  auto receive = [&](const v16f (&a)[4], v16f (&f)[4]) {
    const uint8_t* in = lds + ((size_t)(pos * 2 + h) * 4) * 4 * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const v4f o = *reinterpret_cast<const v4f*>(in + ((i * 4 + e4) * 64 + lane) * 16);
        f[i][4 * e4] = a[i][4 * e4] + o.x + bj;
        f[i][4 * e4 + 1] = a[i][4 * e4 + 1] + o.y + bj;
        f[i][4 * e4 + 2] = a[i][4 * e4 + 2] + o.z + bj;
        f[i][4 * e4 + 3] = a[i][4 * e4 + 3] + o.w + bj;
      }
  };
  v16f c0[4], c1[4], fin[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c0[i] = acc[i][0];
    c1[i] = acc[i][1];
  }
  if (h == 0)
    send(c1);
  else
    send(c0);
  stage_barrier();
  if (h == 0)
    receive(c0, fin);
  else
    receive(c1, fin);
  const int col = col0 + 32 * h + l32;
  if (m_tile + TM <= M && n_tile + TN <= N) {
    // a whole tile (all but the ragged edge): no per-element bounds, one uniform base and
    // fixed row offsets (< 128 N < 2^31: N <= 2^24), and pairs of rows rounded to bf16 by one
    // conversion (RNE).  Y is written once and not read here: non-temporal stores stream it out
    // instead of leaving it dirty in the caches, where the next kernel's reads would wait on
    // its write-back.
    const size_t base = (size_t)row0 * N + col;
    const uint32_t lo = (uint32_t)(4 * hi) * (uint32_t)N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {  // rows e and e + 1 are consecutive (e % 4 in {0, 2})
        const uint32_t o = lo + (uint32_t)(32 * i + 8 * (e >> 2) + (e & 3)) * (uint32_t)N;
        const float v0 = fin[i][e], v1 = fin[i][e + 1];
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
  if (col < No) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < Mo) {
          if constexpr (OUT_FP32)
            reinterpret_cast<float*>(Y)[(size_t)row * No + col] = fin[i][e];
          else
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * No + col] = float_to_bf16_bits(fin[i][e]);
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
    /* four resident stages need more than the default 64 KB of dynamic LDS */                 \
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
  const dim3 grid(((M + f6::TM - 1) / f6::TM) * ((N + f6::TN - 1) / f6::TN));
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
