// Host-side argument validation for the libgqa C ABI. Pure C++ (no HIP
// headers): every rule here runs before anything is enqueued, so it is
// testable on a machine without a GPU.
//
// Rules follow the statement of the problem on the pages: Hq query heads in
// Hkv equal groups (page "TensorRT对Grouped Query Attention的支持进展",
// section "技术演进背景"; non-uniform grouping is rejected), fixed-size
// pages addressed through a page table (same page, section
// "动态形状与KV Cache管理"), NumSplits >= 1 (page
// "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", section
// "核心参数调优：PackGQA与NumSplits的协同舞蹈").
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/gqa.h"

namespace {

constexpr int kMaxSplits = 256;
constexpr int kMaxGridY = 65535;

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_decode_group(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}
bool supported_prefill_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Shape checks common to decode and prefill.
int check_common(int B, int Hq, int Hkv, int D, int P, int max_pages, int num_pages,
                 float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || max_pages <= 0 || num_pages <= 0)
    return GQA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if ((int64_t)B * max_pages > INT32_MAX) return GQA_ERR_INVALID_ARG;
  if (!supported_head_dim(D) || P != 16) return GQA_ERR_UNSUPPORTED;
  if (B > kMaxGridY) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

}  // namespace

extern "C" {

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_LAUNCH: return "kernel launch failed";
    case GQA_ERR_SCRATCH: return "problem needs more than the static scratch buffer holds";
    default: return "unknown status";
  }
}

size_t gqa_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B <= 0 || Hq <= 0 || D <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Hq * num_splits;
  return rows * (size_t)D * sizeof(float) + rows * sizeof(float);
}

int gqa_validate_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* context_lens, const void* out,
                        const float* ws_o, const float* ws_lse, int B, int Hq, int Hkv, int D,
                        int P, int max_pages, int num_pages, int num_splits, float scale,
                        int dtype) {
  if (!q || !k_cache || !v_cache || !page_table || !context_lens || !out)
    return GQA_ERR_INVALID_ARG;
  if (num_splits < 1) return GQA_ERR_INVALID_ARG;
  if (num_splits > 1 && (!ws_o || !ws_lse)) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, D, P, max_pages, num_pages, scale);
  if (st != GQA_OK) return st;
  if (!supported_decode_group(Hq / Hkv)) return GQA_ERR_UNSUPPORTED;
  if (num_splits > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)Hkv * num_splits > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;  // grid.x
  return GQA_OK;
}

}  // extern "C"

namespace {

// Split count of the split path when the balanced entry point takes it: enough splits for
// one workgroup per CU of the 256-CU MI355X and no more (measured with B x Hkv from 1 to 256,
// Hq = 32, T = 1024: fewer splits leave CUs idle, more add combine traffic and shorter
// per-split streams).
int auto_splits(int B, int Hkv) {
  const long units = (long)B * Hkv;
  if (units <= 0) return 1;
  long ns = (256 + units - 1) / units;
  return (int)(ns < 1 ? 1 : (ns > 16 ? 16 : ns));
}

// Bytes of the persistent path's partial slots: 4096 waves x 2 slots of G x D + G floats
// rounded up to whole 128-byte lines.
size_t slot_area_bytes(int G, int D) {
  if (G > 8) return 0;
  const size_t slot_floats = ((size_t)G * D + G + 31) / 32 * 32;
  return (size_t)4096 * 2 * slot_floats * sizeof(float);
}

}  // namespace

extern "C" {

// Route of the balanced entry point. G <= 8: the persistent kernel, except for small problems,
// which run faster on the split path with at least 16 pages per split, provided its partials
// fit in the workspace past the counters: at most 1,024 (sequence, KV head, page) items (any
// G <= 8; measured with T = 1024, Hq = 32 and B from 1 to 256), or 65,536 with one query head
// per KV head, or, for G = 2 and G = 4, at most 16,384 / 8,192 items when the split path takes
// at most 4 splits of page-table rows of at least 16 pages (uniform and ragged batches,
// Hq = 32: the split path at 0.64-1.02 of the persistent kernel's time there, and slower with
// 8 or 16 splits, with 8-page rows, and at G = 8). G >= 16: the split path with auto_splits splits, at least 8 pages per split (with
// T = 1024 and B = 1 or 16, 8 splits were 9-10% faster than 16, whose 4 pages per split give
// each of the 4 waves a single page).
int gqa_decode_balanced_route(int B, int Hq, int Hkv, int D, int max_pages,
                              size_t workspace_bytes) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_pages <= 0 || Hq % Hkv != 0) return -1;
  const int G = Hq / Hkv;
  int ns = auto_splits(B, Hkv);
  if (G > 8) {
    const int cap = max_pages / 8 < 1 ? 1 : max_pages / 8;
    return ns < cap ? ns : cap;
  }
  {
    const long items = (long)B * Hkv * max_pages;
    ns = max_pages / 16 < ns ? max_pages / 16 : ns;
    if (ns < 1) ns = 1;
    const long mid = G == 2 ? 16384 : (G == 4 ? 8192 : 0);  // few splits, rows of 16+ pages
    const bool small = items <= (G == 1 ? 65536 : 1024) ||
                       (items <= mid && ns <= 4 && max_pages >= 16);
    const size_t split_bytes = ns == 1 ? 0 : gqa_decode_workspace_bytes(B, Hq, D, ns);
    if (!small || GQA_BALANCED_WS_RESERVED + split_bytes > workspace_bytes) return 0;
  }
  return ns;
}

// Workspace of the balanced entry point: counters, then per-wave partial slots (G <= 8) or
// the split partials (G >= 16).
size_t gqa_decode_balanced_workspace_bytes(int B, int Hq, int Hkv, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return 0;
  const int G = Hq / Hkv;
  const size_t slot_bytes = slot_area_bytes(G, D);
  const int ns = auto_splits(B, Hkv);
  const size_t split_bytes = G >= 16 && ns > 1 ? gqa_decode_workspace_bytes(B, Hq, D, ns) : 0;
  return GQA_BALANCED_WS_RESERVED + (slot_bytes > split_bytes ? slot_bytes : split_bytes);
}

// Page ids that a call would read or write, checked against the pool on the host: for every
// sequence the first ceil(tokens[b] / P) entries of its row (tokens clamped to
// [0, max_pages * P]) must lie in [0, num_pages).
int gqa_check_page_table(const int32_t* page_table, const int32_t* tokens, int B,
                         int max_pages, int P, int num_pages) {
  if (!page_table || !tokens) return GQA_ERR_INVALID_ARG;
  if (B <= 0 || max_pages <= 0 || P <= 0 || num_pages <= 0) return GQA_ERR_INVALID_ARG;
  if ((int64_t)max_pages * P > INT32_MAX) return GQA_ERR_INVALID_ARG;
  const int cap = max_pages * P;
  for (int b = 0; b < B; ++b) {
    int t = tokens[b];
    t = t < 0 ? 0 : (t > cap ? cap : t);
    const int np = (t + P - 1) / P;
    const int32_t* row = page_table + (size_t)b * max_pages;
    for (int i = 0; i < np; ++i)
      if (row[i] < 0 || row[i] >= num_pages) return GQA_ERR_INVALID_ARG;
  }
  return GQA_OK;
}

int gqa_validate_prefill(const void* q, const void* k, const void* v, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const void* out, int B,
                         int S, int Hq, int Hkv, int D, int P, int max_pages, int num_pages,
                         float scale, int dtype) {
  if (!q || !k || !v || !k_cache || !v_cache || !page_table || !out) return GQA_ERR_INVALID_ARG;
  if (S <= 0) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, D, P, max_pages, num_pages, scale);
  if (st != GQA_OK) return st;
  if ((int64_t)max_pages * P < S) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (D != 128) return GQA_ERR_UNSUPPORTED;
  if (!supported_prefill_group(Hq / Hkv)) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)S * Hq > INT32_MAX / 256) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

int gqa_validate_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                            float k_scale, float v_scale, const int32_t* page_table,
                            const int32_t* context_lens, const void* out, int B, int Hq, int Hkv,
                            int D, int P, int max_pages, int num_pages, float scale,
                            int kv_dtype) {
  if (kv_dtype != GQA_FP8_E4M3 && kv_dtype != GQA_FP8_E5M2) return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f)
    return GQA_ERR_INVALID_ARG;
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                               nullptr, B, Hq, Hkv, D, P, max_pages, num_pages, 1, scale,
                               GQA_BF16);
  if (st != GQA_OK) return st;
  if (D != 128 || Hq / Hkv > 8) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

int gqa_validate_prefill_paged(const void* q, const void* k, const void* v, const void* k_cache,
                               const void* v_cache, const int32_t* page_table,
                               const int32_t* past_lens, const int32_t* new_lens, const void* out,
                               int B, int S, int Hq, int Hkv, int D, int P, int max_pages,
                               int num_pages, float scale, int dtype) {
  if (!past_lens || !new_lens) return GQA_ERR_INVALID_ARG;
  if (!q || !k || !v || !k_cache || !v_cache || !page_table || !out) return GQA_ERR_INVALID_ARG;
  if (S <= 0) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  int st = check_common(B, Hq, Hkv, D, P, max_pages, num_pages, scale);
  if (st != GQA_OK) return st;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (D != 128) return GQA_ERR_UNSUPPORTED;
  if (!supported_prefill_group(Hq / Hkv)) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)S * Hq > INT32_MAX / 256) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * P > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

int gqa_validate_combine(const float* ws_o, const float* ws_lse, const void* out, int B, int Hq,
                         int D, int num_splits, int out_dtype) {
  if (!ws_o || !ws_lse || !out) return GQA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || D <= 0 || num_splits < 1) return GQA_ERR_INVALID_ARG;
  if (out_dtype != GQA_F32 && out_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (!supported_head_dim(D)) return GQA_ERR_UNSUPPORTED;
  if (num_splits > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

}  // extern "C"
