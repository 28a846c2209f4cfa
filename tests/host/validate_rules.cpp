// Host-only rules of the libgqa C ABI (argument validation, workspace sizes, the balanced
// route, the page-id check), exercised in a plain C++ program so that they can be built with
// AddressSanitizer and UndefinedBehaviorSanitizer. Links validate.cpp only: no GPU, no HIP.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "../../include/gqa.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static char fake_buf[64];
static const void* F = fake_buf;  // never dereferenced: the rules only test for null

static int vd(int B, int Hq, int Hkv, int D, int P, int mp, int np, int ns, float scale,
              int dtype, bool ws = false) {
  return gqa_validate_decode(F, F, F, (const int32_t*)F, (const int32_t*)F, F,
                             ws ? (const float*)F : nullptr, ws ? (const float*)F : nullptr, B,
                             Hq, Hkv, D, P, mp, np, ns, scale, dtype);
}

int main() {
  // decode
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 1, 0.125f, GQA_BF16) == GQA_OK);
  for (int G : {1, 2, 4, 8, 16, 32}) EXPECT(vd(2, 32, 32 / G, 128, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_OK);
  EXPECT(vd(2, 6, 4, 128, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(0, 8, 2, 128, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(2, 8, 2, 128, 16, -1, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 4, 0.1f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 4, 0.1f, GQA_BF16, true) == GQA_OK);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 1, std::nanf(""), GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 1, std::numeric_limits<float>::infinity(), GQA_BF16) ==
         GQA_ERR_INVALID_ARG);
  EXPECT(vd(2, 8, 2, 96, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(vd(2, 8, 2, 128, 32, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(vd(2, 12, 4, 128, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 1000, 0.1f, GQA_BF16, true) == GQA_ERR_UNSUPPORTED);
  // sizes that would overflow 32-bit products are refused, not wrapped
  EXPECT(vd(65535, 8, 2, 128, 16, 1 << 20, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(vd(70000, 8, 2, 128, 16, 4, 8, 1, 0.1f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(vd(2, 8, 2, 128, 16, 4, 8, 1 << 30, 0.1f, GQA_BF16, true) == GQA_ERR_UNSUPPORTED);

  // prefill
  const int32_t* pt = (const int32_t*)F;
  EXPECT(gqa_validate_prefill(F, F, F, F, F, pt, F, 4, 2048, 32, 8, 128, 16, 128, 600, 0.088f,
                              GQA_BF16) == GQA_OK);
  EXPECT(gqa_validate_prefill(F, F, F, F, F, pt, F, 4, 2048, 32, 8, 128, 16, 127, 600, 0.088f,
                              GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_prefill(F, F, F, F, F, pt, F, 4, 1 << 30, 32, 8, 128, 16, 1 << 27, 600,
                              0.088f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_validate_prefill_paged(F, F, F, F, F, pt, pt, pt, F, 4, 512, 32, 8, 128, 16,
                                    1 << 27, 512, 0.088f, GQA_BF16) == GQA_ERR_UNSUPPORTED);
  EXPECT(gqa_validate_prefill_paged(F, F, F, F, F, pt, nullptr, pt, F, 4, 512, 32, 8, 128, 16,
                                    8, 512, 0.088f, GQA_BF16) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_decode_fp8(F, F, F, 0.01f, 0.02f, pt, pt, F, 4, 32, 8, 128, 16, 64, 4096,
                                 0.088f, GQA_FP8_E4M3) == GQA_OK);
  EXPECT(gqa_validate_decode_fp8(F, F, F, 0.0f, 0.02f, pt, pt, F, 4, 32, 8, 128, 16, 64, 4096,
                                 0.088f, GQA_FP8_E4M3) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_combine((const float*)F, (const float*)F, F, 4, 32, 128, 8, GQA_BF16) ==
         GQA_OK);
  EXPECT(gqa_validate_combine((const float*)F, (const float*)F, F, 1 << 20, 1 << 12, 128, 8,
                              GQA_BF16) == GQA_ERR_UNSUPPORTED);

  // workspace sizes, including shapes whose products exceed 32 bits
  EXPECT(gqa_decode_workspace_bytes(8, 32, 128, 16) == (size_t)8 * 32 * 16 * 129 * 4);
  EXPECT(gqa_decode_workspace_bytes(65535, 4096, 128, 256) ==
         (size_t)65535 * 4096 * 256 * 129 * 4);
  EXPECT(gqa_decode_balanced_workspace_bytes(64, 32, 8, 128) ==
         GQA_BALANCED_WS_RESERVED + (size_t)4096 * 2 * 544 * 4);
  EXPECT(gqa_decode_balanced_workspace_bytes(0, 32, 8, 128) == 0);
  EXPECT(gqa_decode_balanced_workspace_bytes(64, 32, 8, 128) <= GQA_NOALLOC_SCRATCH_BYTES);
  EXPECT(gqa_decode_balanced_workspace_bytes(1, 32, 1, 128) <= GQA_NOALLOC_SCRATCH_BYTES);

  // route
  EXPECT(gqa_decode_balanced_route(1, 32, 8, 128, 128, 1 << 30) >= 1);
  EXPECT(gqa_decode_balanced_route(1, 32, 8, 128, 129, 1 << 30) == 0);
  EXPECT(gqa_decode_balanced_route(1, 1, 1, 128, 65537, 1 << 30) == 0);
  EXPECT(gqa_decode_balanced_route(65535, 32, 32, 128, 1 << 16, 1 << 30) == 0);
  EXPECT(gqa_decode_balanced_route(1, 32, 1, 128, 64, 1 << 30) == 8);     // >= 8 pages per split
  EXPECT(gqa_decode_balanced_route(1, 32, 1, 128, 4096, 1 << 30) == 16);
  EXPECT(gqa_decode_balanced_route(0, 32, 8, 128, 64, 1 << 30) == -1);

  // page-id check over host arrays
  std::vector<int32_t> table = {3, 0, -1, 99, 1, 2, 5, 7};
  std::vector<int32_t> tokens = {32, 64};
  EXPECT(gqa_check_page_table(table.data(), tokens.data(), 2, 4, 16, 8) == GQA_OK);
  tokens[0] = 33;
  EXPECT(gqa_check_page_table(table.data(), tokens.data(), 2, 4, 16, 8) == GQA_ERR_INVALID_ARG);
  tokens[0] = std::numeric_limits<int32_t>::max();
  tokens[1] = std::numeric_limits<int32_t>::min();
  EXPECT(gqa_check_page_table(table.data(), tokens.data(), 2, 4, 16, 8) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_check_page_table(table.data(), tokens.data(), 2, 1 << 30, 16, 8) ==
         GQA_ERR_INVALID_ARG);  // max_pages * P beyond int32: refused before any read
  EXPECT(gqa_check_page_table(nullptr, tokens.data(), 2, 4, 16, 8) == GQA_ERR_INVALID_ARG);

  for (int st = -1; st <= 5; ++st) EXPECT(gqa_status_string(st) != nullptr);
  if (failures) return 1;
  std::printf("host rules: all checks passed\n");
  return 0;
}
