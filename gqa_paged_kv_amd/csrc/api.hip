// extern "C" entry points of libgqa: validate on the host, then enqueue kernels on
// the caller's stream. No allocation and no synchronisation (a build with GQA_DEBUG defined
// checks page ids on the host first, which synchronises the stream).
#include <algorithm>
#include <hip/hip_runtime.h>

#include "../../include/gqa.h"

namespace gqa {
struct bf16_t;
int launch_decode_paged(const void* q, const void* k, const void* v, const int32_t* pt,
                        const int32_t* lens, void* out, float* ws_o, float* ws_lse, int B,
                        int Hq, int Hkv, int D, int max_pages, int ns, float scale, int dtype,
                        hipStream_t s);
int launch_combine(const float* ws_o, const float* ws_lse, void* out, int B, int Hq, int D,
                   int ns, int dtype, hipStream_t s);
int launch_gather(const void* cache, const int32_t* pt, const int32_t* lens, void* dst, int B,
                  int Hkv, int D, int P, int max_pages, int dtype, hipStream_t s);
int launch_decode_balanced(const void* q, const void* k, const void* v, const int32_t* pt,
                           const int32_t* lens, void* out, void* slots, int B, int Hq, int Hkv,
                           int D, int max_pages, float scale, int dtype, hipStream_t s);
int launch_decode_append(const void* q, const void* k_new, const void* v_new, void* k, void* v,
                         const int32_t* pt, const int32_t* lens, void* out, void* ws, int B,
                         int Hq, int Hkv, int D, int max_pages, float scale, int dtype,
                         hipStream_t s);
int launch_decode_balanced_fp8(const void* q, const void* k, const void* v, float k_scale,
                               float v_scale, const int32_t* pt, const int32_t* lens, void* out,
                               void* ws, int B, int Hq, int Hkv, int D, int max_pages,
                               float scale, int kv_dtype, hipStream_t s);
int noalloc_scratch(void** ptr, hipStream_t s);
int launch_prefill(const void* q, const void* k, const void* v, void* out, void* k_cache,
                   void* v_cache, const int32_t* page_table, int max_pages, int B, int S, int Hq,
                   int Hkv, int D, float scale, hipStream_t s);
int launch_prefill_paged(const void* q, const void* k, const void* v, void* out, void* k_cache,
                         void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                         const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv,
                         int D, float scale, hipStream_t s);
}  // namespace gqa


#ifdef GQA_DEBUG
#include <vector>
// Debug build: before anything is enqueued, the page table and the per-sequence lengths are
// copied to the host (after the work already queued on `stream`, which may have written
// them) and every page id the call would touch is checked against the pool by
// gqa_check_page_table. kind 0: decode over lens[b] tokens; 1: decode with the step's token
// appended (lens[b] clamped to max_pages * P - 1, plus one); 2: prefill of S tokens per
// sequence; 3: chunked prefill, past (lens) plus new (lens2) tokens.
namespace {
int debug_check_pages(const int32_t* pt, const int32_t* lens, const int32_t* lens2, int kind,
                      int S, int B, int max_pages, int P, int num_pages, hipStream_t s) {
  std::vector<int32_t> h_pt((size_t)B * max_pages), a(B, 0), n(B, 0), tok(B, 0);
  if (hipMemcpyAsync(h_pt.data(), pt, h_pt.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return GQA_ERR_LAUNCH;
  if (lens && hipMemcpyAsync(a.data(), lens, (size_t)B * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return GQA_ERR_LAUNCH;
  if (lens2 && hipMemcpyAsync(n.data(), lens2, (size_t)B * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return GQA_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return GQA_ERR_LAUNCH;
  const int cap = max_pages * P;
  for (int b = 0; b < B; ++b) {
    const int t = std::min(std::max(a[b], 0), cap);
    if (kind == 0) tok[b] = t;
    if (kind == 1) tok[b] = std::min(std::max(a[b], 0), cap - 1) + 1;
    if (kind == 2) tok[b] = S;
    if (kind == 3) tok[b] = t + std::min(std::max(n[b], 0), std::min(S, cap - t));
  }
  return gqa_check_page_table(h_pt.data(), tok.data(), B, max_pages, P, num_pages);
}
}  // namespace
#define GQA_DEBUG_CHECK_PAGES(pt, lens, lens2, kind, S, B, mp, P, np, stream)                   \
  do {                                                                                          \
    const int st_ = debug_check_pages(pt, lens, lens2, kind, S, B, mp, P, np,                   \
                                      (hipStream_t)(stream));                                   \
    if (st_ != GQA_OK) return st_;                                                              \
  } while (0)
#else
#define GQA_DEBUG_CHECK_PAGES(pt, lens, lens2, kind, S, B, mp, P, np, stream) \
  do {                                                                       \
  } while (0)
#endif

extern "C" {

int gqa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, const int32_t* context_lens, void* out,
                     float* ws_o, float* ws_lse, int B, int Hq, int Hkv, int D, int P,
                     int max_pages, int num_pages, int num_splits, float scale, int dtype,
                     void* stream) {
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, ws_o, ws_lse,
                               B, Hq, Hkv, D, P, max_pages, num_pages, num_splits, scale, dtype);
  if (st != GQA_OK) return st;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 0, 0, B, max_pages, P, num_pages, stream);
  hipStream_t s = (hipStream_t)stream;
  st = gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out, ws_o, ws_lse,
                                B, Hq, Hkv, D, max_pages, num_splits, scale, dtype, s);
  if (st != GQA_OK || num_splits == 1) return st;
  return gqa::launch_combine(ws_o, ws_lse, out, B, Hq, D, num_splits, dtype, s);
}

}  // extern "C"

// The balanced decode on a validated call with `workspace` (workspace_bytes of it usable).
static int decode_balanced_on(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* context_lens, void* out,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int D, int max_pages, float scale, int dtype, hipStream_t s) {
  char* data = (char*)workspace;
  const int ns = gqa_decode_balanced_route(B, Hq, Hkv, D, max_pages, workspace_bytes);
  if (ns == 0)
    return gqa::launch_decode_balanced(q, k_cache, v_cache, page_table, context_lens, out, data,
                                       B, Hq, Hkv, D, max_pages, scale, dtype, s);
  if (ns == 1)
    return gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                                    nullptr, B, Hq, Hkv, D, max_pages, 1, scale, dtype, s);
  // the split partials start past the persistent path's counters
  float* ws_o = (float*)(data + GQA_BALANCED_WS_RESERVED);
  float* ws_lse = ws_o + (size_t)B * Hq * ns * D;
  const int st = gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out,
                                          ws_o, ws_lse, B, Hq, Hkv, D, max_pages, ns, scale,
                                          dtype, s);
  if (st != GQA_OK) return st;
  return gqa::launch_combine(ws_o, ws_lse, out, B, Hq, D, ns, dtype, s);
}

extern "C" {

int gqa_decode_paged_balanced(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* context_lens, void* out,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int D, int P, int max_pages, int num_pages, float scale, int dtype,
                              void* stream) {
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                               nullptr, B, Hq, Hkv, D, P, max_pages, num_pages, 1, scale, dtype);
  if (st != GQA_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255) != 0) return GQA_ERR_INVALID_ARG;
  if (workspace_bytes < gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D)) return GQA_ERR_INVALID_ARG;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 0, 0, B, max_pages, P, num_pages, stream);
  return decode_balanced_on(q, k_cache, v_cache, page_table, context_lens, out, workspace,
                            workspace_bytes, B, Hq, Hkv, D, max_pages, scale, dtype,
                            (hipStream_t)stream);
}

int gqa_decode_paged_balanced_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* page_table, const int32_t* context_lens,
                                      void* out, int B, int Hq, int Hkv, int D, int P,
                                      int max_pages, int num_pages, float scale, int dtype,
                                      void* stream) {
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                               nullptr, B, Hq, Hkv, D, P, max_pages, num_pages, 1, scale, dtype);
  if (st != GQA_OK) return st;
  if (gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D) > GQA_NOALLOC_SCRATCH_BYTES)
    return GQA_ERR_SCRATCH;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 0, 0, B, max_pages, P, num_pages, stream);
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  st = gqa::noalloc_scratch(&ws, s);
  if (st != GQA_OK) return st;
  return decode_balanced_on(q, k_cache, v_cache, page_table, context_lens, out, ws,
                            GQA_NOALLOC_SCRATCH_BYTES, B, Hq, Hkv, D, max_pages, scale, dtype, s);
}

int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                      void* out, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                      int D, int P, int max_pages, int num_pages, float scale, int dtype,
                      void* stream) {
  if (!k_new || !v_new) return GQA_ERR_INVALID_ARG;
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                               nullptr, B, Hq, Hkv, D, P, max_pages, num_pages, 1, scale, dtype);
  if (st != GQA_OK) return st;
  if (Hq / Hkv > 8) return GQA_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace & 255) != 0) return GQA_ERR_INVALID_ARG;
  if (workspace_bytes < gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D)) return GQA_ERR_INVALID_ARG;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 1, 0, B, max_pages, P, num_pages, stream);
  return gqa::launch_decode_append(q, k_new, v_new, k_cache, v_cache, page_table, context_lens,
                                   out, workspace, B, Hq, Hkv, D, max_pages, scale, dtype,
                                   (hipStream_t)stream);
}

int gqa_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                         float v_scale, const int32_t* page_table, const int32_t* context_lens,
                         void* out, void* workspace, size_t workspace_bytes, int B, int Hq,
                         int Hkv, int D, int P, int max_pages, int num_pages, float scale,
                         int kv_dtype, void* stream) {
  int st = gqa_validate_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, page_table,
                                   context_lens, out, B, Hq, Hkv, D, P, max_pages, num_pages,
                                   scale, kv_dtype);
  if (st != GQA_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255) != 0) return GQA_ERR_INVALID_ARG;
  if (workspace_bytes < gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D)) return GQA_ERR_INVALID_ARG;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 0, 0, B, max_pages, P, num_pages, stream);
  return gqa::launch_decode_balanced_fp8(q, k_cache, v_cache, k_scale, v_scale, page_table,
                                         context_lens, out, workspace, B, Hq, Hkv, D, max_pages,
                                         scale, kv_dtype, (hipStream_t)stream);
}

int gqa_combine_splits(const float* ws_o, const float* ws_lse, void* out, int B, int Hq, int D,
                       int num_splits, int out_dtype, void* stream) {
  int st = gqa_validate_combine(ws_o, ws_lse, out, B, Hq, D, num_splits, out_dtype);
  if (st != GQA_OK) return st;
  return gqa::launch_combine(ws_o, ws_lse, out, B, Hq, D, num_splits, out_dtype,
                             (hipStream_t)stream);
}

int gqa_prefill_causal(const void* q, const void* k, const void* v, void* k_cache,
                       void* v_cache, const int32_t* page_table, void* out, int B, int S,
                       int Hq, int Hkv, int D, int P, int max_pages, int num_pages,
                       float scale, int dtype, void* stream) {
  int st = gqa_validate_prefill(q, k, v, k_cache, v_cache, page_table, out, B, S, Hq, Hkv, D, P,
                                max_pages, num_pages, scale, dtype);
  if (st != GQA_OK) return st;
  GQA_DEBUG_CHECK_PAGES(page_table, nullptr, nullptr, 2, S, B, max_pages, P, num_pages, stream);
  // one kernel: attention plus the append of the new K/V rows into the cache
  return gqa::launch_prefill(q, k, v, out, k_cache, v_cache, page_table, max_pages, B, S, Hq, Hkv,
                             D, scale, (hipStream_t)stream);
}

int gqa_prefill_paged(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      const int32_t* page_table, const int32_t* past_lens,
                      const int32_t* new_lens, void* out, int B, int S, int Hq, int Hkv, int D,
                      int P, int max_pages, int num_pages, float scale, int dtype, void* stream) {
  int st = gqa_validate_prefill_paged(q, k, v, k_cache, v_cache, page_table, past_lens, new_lens,
                                      out, B, S, Hq, Hkv, D, P, max_pages, num_pages, scale, dtype);
  if (st != GQA_OK) return st;
  GQA_DEBUG_CHECK_PAGES(page_table, past_lens, new_lens, 3, S, B, max_pages, P, num_pages, stream);
  return gqa::launch_prefill_paged(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens,
                                   max_pages, B, S, Hq, Hkv, D, scale, (hipStream_t)stream);
}

int gqa_gather_paged(const void* cache, const int32_t* page_table, const int32_t* context_lens,
                     void* dst, int B, int Hkv, int D, int P, int max_pages, int num_pages,
                     int dtype, void* stream) {
  if (!cache || !page_table || !context_lens || !dst) return GQA_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || max_pages <= 0 || num_pages <= 0)
    return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || P != 16 || B > 65535) return GQA_ERR_UNSUPPORTED;
  GQA_DEBUG_CHECK_PAGES(page_table, context_lens, nullptr, 0, 0, B, max_pages, P, num_pages, stream);
  return gqa::launch_gather(cache, page_table, context_lens, dst, B, Hkv, D, P, max_pages, dtype,
                            (hipStream_t)stream);
}

}  // extern "C"
