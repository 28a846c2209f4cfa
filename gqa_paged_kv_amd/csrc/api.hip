// extern "C" entry points of libgqa: validate on the host, then enqueue kernels on
// the caller's stream. No allocation, no synchronisation, no global state.
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
int launch_prefill(const void* q, const void* k, const void* v, void* out, void* k_cache,
                   void* v_cache, const int32_t* page_table, int max_pages, int B, int S, int Hq,
                   int Hkv, int D, float scale, hipStream_t s);
int launch_prefill_paged(const void* q, const void* k, const void* v, void* out, void* k_cache,
                         void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                         const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv,
                         int D, float scale, hipStream_t s);
}  // namespace gqa

extern "C" int gqa_balanced_auto_splits(int B, int Hkv);

extern "C" {

int gqa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, const int32_t* context_lens, void* out,
                     float* ws_o, float* ws_lse, int B, int Hq, int Hkv, int D, int P,
                     int max_pages, int num_pages, int num_splits, float scale, int dtype,
                     void* stream) {
  int st = gqa_validate_decode(q, k_cache, v_cache, page_table, context_lens, out, ws_o, ws_lse,
                               B, Hq, Hkv, D, P, max_pages, num_pages, num_splits, scale, dtype);
  if (st != GQA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out, ws_o, ws_lse,
                                B, Hq, Hkv, D, max_pages, num_splits, scale, dtype, s);
  if (st != GQA_OK || num_splits == 1) return st;
  return gqa::launch_combine(ws_o, ws_lse, out, B, Hq, D, num_splits, dtype, s);
}

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
  hipStream_t s = (hipStream_t)stream;
  char* data = (char*)workspace;
  const int G = Hq / Hkv;
  int ns = gqa_balanced_auto_splits(B, Hkv);
  if (G <= 8) {
    // Small problems (at most 1,024 (sequence, KV head, page) items, or 65,536 with one query
    // head per KV head) run faster on the split path, with at least 16 pages per split, whose
    // partials then fit in the slot area of the workspace; measured with T = 1024, Hq = 32 and
    // B from 1 to 256.
    const long items = (long)B * Hkv * max_pages;
    const bool small = items <= (G == 1 ? 65536 : 1024);
    ns = std::max(1, std::min(ns, max_pages / 16));
    const size_t split_bytes = ns == 1 ? 0 : gqa_decode_workspace_bytes(B, Hq, D, ns);
    if (!small || GQA_BALANCED_WS_RESERVED + split_bytes > workspace_bytes)
      return gqa::launch_decode_balanced(q, k_cache, v_cache, page_table, context_lens, out, data,
                                         B, Hq, Hkv, D, max_pages, scale, dtype, s);
  }
  if (ns == 1)
    return gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out, nullptr,
                                    nullptr, B, Hq, Hkv, D, max_pages, 1, scale, dtype, s);
  // the split partials start past the persistent path's counters, which stay zero
  float* ws_o = (float*)(data + GQA_BALANCED_WS_RESERVED);
  float* ws_lse = ws_o + (size_t)B * Hq * ns * D;
  st = gqa::launch_decode_paged(q, k_cache, v_cache, page_table, context_lens, out, ws_o, ws_lse,
                                B, Hq, Hkv, D, max_pages, ns, scale, dtype, s);
  if (st != GQA_OK) return st;
  return gqa::launch_combine(ws_o, ws_lse, out, B, Hq, D, ns, dtype, s);
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
  return gqa::launch_gather(cache, page_table, context_lens, dst, B, Hkv, D, P, max_pages, dtype,
                            (hipStream_t)stream);
}

}  // extern "C"
