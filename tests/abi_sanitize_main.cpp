// Host-only driver for the C ABI's validation paths, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi_cpu.py (a CPU build; no call here reaches a
// kernel launch).  Every entry point is called with NULL, misaligned, out-of-range and
// overflowing arguments and must return the documented status without a sanitizer report;
// the size queries are called with extreme sizes and must not overflow.  Exits 0 when every
// check holds, 1 otherwise (the failing check is printed).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "svdq.h"

static int failures = 0;

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main() {
  // fake device addresses: never dereferenced, because every call below fails validation
  void* F = reinterpret_cast<void*>(0x10000);
  void* O = reinterpret_cast<void*>(0x10008);  // 8-byte aligned only
  auto u8 = [](void* p) { return static_cast<uint8_t*>(p); };
  auto u16 = [](void* p) { return static_cast<uint16_t*>(p); };
  auto f32 = [](void* p) { return static_cast<float*>(p); };
  auto i8 = [](void* p) { return static_cast<int8_t*>(p); };
  auto i32 = [](void* p) { return static_cast<int32_t*>(p); };

  EXPECT(svdq_abi_version() == SVDQ_ABI_VERSION);
  for (int s = -1; s <= 6; ++s) EXPECT(std::strlen(svdq_status_str(s)) > 0);
  EXPECT(std::strcmp(svdq_status_str(INT_MIN), "unknown status") == 0);

  // ---- weight packing and the factor relayout
  EXPECT(svdq_pack_weights(f32(F), 100, 8, u8(F), u16(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_pack_weights(f32(F), INT_MIN, 8, u8(F), u16(F), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_weights(f32(F), 64, INT_MIN, u8(F), u16(F), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_weights(f32(F), INT_MAX / 64 * 64, INT_MAX, u8(F), u16(F), nullptr) ==
         SVDQ_ESHAPE);
  EXPECT(svdq_pack_weights(f32(O), 64, 8, u8(F), u16(F), nullptr) == SVDQ_EALIGN);
  EXPECT(svdq_pack_weights_e3m2(nullptr, 64, 8, u8(F), u16(F), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_lowrank(u16(F), INT_MAX / 64 * 64, 16, u16(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_pack_lowrank(u16(F), 128, INT_MAX, u16(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_pack_lowrank(u16(F), 128, INT_MIN, u16(F), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_lowrank_up(u16(F), 16, INT_MAX, u16(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_pack_lowrank_up(u16(F), INT_MIN, 64, u16(F), nullptr) == SVDQ_EINVAL);

  // ---- activation pass (three containers)
  EXPECT(svdq_quantize_act(u16(F), f32(F), u16(F), INT_MAX, INT_MAX / 64 * 64, 16, u8(F), u16(F),
                           f32(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_quantize_act(u16(F), f32(F), u16(F), INT_MIN, 128, 16, u8(F), u16(F), f32(F),
                           nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_quantize_act_e3m2(u16(F), f32(F), nullptr, 4, 128, 16, u8(F), u16(F), f32(F),
                                nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_quantize_act_a8(u16(O), f32(F), u16(F), 4, 128, 16, i8(F), u16(F), f32(F),
                              nullptr) == SVDQ_EALIGN);
  EXPECT(svdq_quantize_act(u16(F), f32(F), u16(F), 0, 128, 16, u8(F), u16(F), f32(F), nullptr) ==
         SVDQ_OK);

  // ---- GEMMs and partials
  const int Ks = INT_MAX / 64 * 64;
  EXPECT(svdq_w4a4_gemm(u8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, INT_MAX, 1, 64, 0,
                        F, SVDQ_OUT_BF16, nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_w4a4_gemm(u8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, 8, INT_MAX, 64, 0,
                        F, SVDQ_OUT_BF16, nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_w4a4_gemm_e3m2(u8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, 8, 8, Ks, 0,
                             F, SVDQ_OUT_BF16, nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_w4a4_gemm(u8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, 8, 8, 128, 16, F,
                        7, nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_w4a8_gemm(i8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, 8, 8, 128, 16, O,
                        SVDQ_OUT_FP32, nullptr) == SVDQ_EALIGN);
  EXPECT(svdq_w4a4_partials(u8(F), u8(F), 8, 8, 96, i32(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(svdq_w4a4_partials_e3m2(u8(F), u8(F), INT_MIN, 8, 128, i32(F), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_w4a8_partials(i8(F), u8(F), 8, 8, 128, nullptr, nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_w4a4_gemm(u8(F), u16(F), f32(F), u8(F), u16(F), u16(F), nullptr, 0, 8, 128, 16, F,
                        SVDQ_OUT_BF16, nullptr) == SVDQ_OK);

  // ---- size queries at the ends of the int range
  EXPECT(svdq_e3m2_bytes(INT_MAX, 64) > 0);
  EXPECT(svdq_e3m2_bytes(INT_MAX, Ks) > 0);
  EXPECT(svdq_e3m2_bytes(INT_MIN, 64) == 0);
  EXPECT(kv_int8_workspace_bytes(INT_MAX, 8) > 0);
  EXPECT(kv_int8_workspace_bytes(INT_MAX, INT_MAX / 8 * 8) > 0);
  EXPECT(kv_int8_workspace_bytes(INT_MIN, 8) == 0);
  EXPECT(kv_int8_attention_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128) > 0);
  EXPECT(kv_int8_attention_workspace_bytes(1, INT_MIN, 1, 64) == 0);

  // ---- KV cache
  EXPECT(kv_int8_quant(u16(F), INT_MAX, 8, u8(F), f32(F), u8(F), F, nullptr) == SVDQ_ESHAPE);
  EXPECT(kv_int8_quant(u16(F), 16, INT_MAX, u8(F), f32(F), u8(F), F, nullptr) == SVDQ_ESHAPE);
  EXPECT(kv_int8_quant(u16(F), INT_MIN, 8, u8(F), f32(F), u8(F), F, nullptr) == SVDQ_EINVAL);
  EXPECT(kv_int8_quant_pair(u16(F), u16(F), 16, 16, u8(F), f32(F), u8(F), u8(F), f32(O), u8(F),
                            F, nullptr) == SVDQ_EALIGN);
  EXPECT(kv_int8_quant_pair(u16(F), u16(F), INT_MAX, INT_MAX / 8 * 8, u8(F), f32(F), u8(F), u8(F),
                            f32(F), u8(F), F, nullptr) == SVDQ_ESHAPE);
  EXPECT(kv_int8_quant_pair_noalloc(u16(F), u16(F), 65536, 4096, u8(F), f32(F), u8(F), u8(F),
                                    f32(F), u8(F), nullptr) == SVDQ_ESHAPE);
  EXPECT(std::strstr(svdq_last_error(), "16777216") != nullptr);
  EXPECT(kv_int8_dequant(u8(F), f32(F), u8(F), 16, INT_MIN, u16(F), nullptr) == SVDQ_EINVAL);
  EXPECT(kv_int8_attention(u16(F), u8(F), f32(F), u8(F), u8(F), f32(F), u8(F), INT_MAX, INT_MAX,
                           INT_MAX, 128, 0.1f, u16(F), F, nullptr) == SVDQ_ESHAPE);
  EXPECT(kv_int8_attention(u16(F), u8(F), f32(F), u8(F), u8(F), f32(F), u8(F), 1, 16, 4, 64,
                           1.0f / 0.0f, u16(F), F, nullptr) == SVDQ_EINVAL);

  // the last-error message is bounded and NUL-terminated
  EXPECT(std::strlen(svdq_last_error()) < 256);

  if (failures) std::fprintf(stderr, "%d check(s) failed\n", failures);
  else std::printf("all ABI validation checks passed\n");
  return failures ? 1 : 0;
}
