/*
 * gqa.h -- C ABI of libgqa: fused grouped-query attention over a paged KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * What is computed (page "TensorRT-LLM与TensorRT核心差异解析", chapter 4,
 * section 4.1 and section 4.2.1): for every query row, out = softmax(scale *
 * q K^T) V evaluated tile by tile on chip, so no score matrix ever reaches
 * memory and only the output is written. Grouping (page "TensorRT对Grouped
 * Query Attention的支持进展", section "技术演进背景"): Hq query heads are
 * split into Hkv contiguous groups of G = Hq / Hkv heads; query head h reads
 * KV head h / G. K/V are never expanded to Hq heads (the repeat_kv of section
 * "图优化与算子融合" is never materialised).
 *
 * Paged cache (same page, section "动态形状与KV Cache管理"; page
 * "TensorRT-LLM与TensorRT核心差异解析" section 4.2.2): the caller owns a pool
 * of fixed-size pages and passes, per call, the physical page ids of each
 * sequence. Token t of sequence b lives in physical page page_table[b][t / P]
 * at slot t % P. Pool layout, for K and for V separately:
 *     cache[num_pages][Hkv][P][D]      (one (page, kv head) block is P*D
 *                                        contiguous elements)
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller. The library never
 *     allocates, frees or synchronises (a build with GQA_DEBUG defined
 *     synchronises the stream to check page ids, see gqa_check_page_table).
 *     Its only state is process-wide and thread-safe: a per-device cache of
 *     the persistent decode grid (an occupancy query made on the first call on
 *     each device) and the epoch counter of the balanced-decode workspaces.
 *     Calls from several host threads are safe when they use different
 *     workspaces.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and runs asynchronously; the return value reports
 *     host-side argument validation and the launch only. A device fault (for
 *     example a page id outside [0, num_pages)) surfaces at the caller's next
 *     synchronisation.
 *   - Tensors are dense and row-major in the layouts given below.
 *   - page_table and context_lens are int32. Only the first ceil(T_b / P)
 *     entries of a page-table row are read; later entries may hold anything.
 *     Cache slots that no live token owns are never read into the result
 *     (they may hold NaN).
 *   - Supported: D in {64, 128}; P == 16; G in {1, 2, 4, 8, 16, 32} for
 *     decode and {1, 2, 4, 8} for prefill; dtype GQA_F32 or GQA_BF16 for
 *     decode, GQA_BF16 for prefill. Accumulation is fp32 throughout.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, Hq % Hkv != 0, ... */
  GQA_ERR_UNSUPPORTED = 2, /* valid but not built: D, P, G or dtype outside the supported set */
  GQA_ERR_LAUNCH = 3,      /* the HIP runtime refused the kernel launch */
  GQA_ERR_SCRATCH = 4      /* the allocation-free entry point's static buffer is too small */
} gqa_status;

/* Bytes at the start of a balanced-decode workspace that hold 64-bit counters. They must be
 * zero before the first call that uses the workspace; every completed call leaves them zero,
 * and every call tags them with a new epoch, so a call that never completed leaves nothing
 * that a later call would count. */
#define GQA_BALANCED_WS_RESERVED 98304

typedef enum {
  GQA_F32 = 0,
  GQA_BF16 = 1,
  GQA_FP8_E4M3 = 2, /* 8-bit float, 4 exponent bits (bias 7), 3 mantissa bits, no inf; cache only */
  GQA_FP8_E5M2 = 3  /* 8-bit float, 5 exponent bits (bias 15), 2 mantissa bits; cache only */
} gqa_dtype;

/*
 * Single-token decode over a paged cache, optionally split along the context
 * (NumSplits: page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践",
 * section "核心参数调优：PackGQA与NumSplits的协同舞蹈").
 *
 *   q            [B][Hq][D]              dtype
 *   k_cache      [num_pages][Hkv][P][D]  dtype
 *   v_cache      [num_pages][Hkv][P][D]  dtype
 *   page_table   [B][max_pages]          int32 physical page ids
 *   context_lens [B]                     int32 T_b; clamped to max_pages*P;
 *                                        T_b <= 0 gives a zero output
 *   out          [B][Hq][D]              dtype; out[b][h] = softmax(scale *
 *                                        q[b][h] . K_b^T) V_b over tokens
 *                                        0 .. T_b-1 (no mask)
 *   ws_o, ws_lse fp32 [B][Hq][num_splits][D] and [B][Hq][num_splits];
 *                may be NULL iff num_splits == 1.
 *   num_splits   NS >= 1. Split s of sequence b covers logical pages
 *                [s*c, min((s+1)*c, np_b)), c = ceil(np_b / NS),
 *                np_b = ceil(T_b / P). With NS > 1 the kernel writes, per
 *                split, the normalised partial output (ws_o) and the
 *                natural-log log-sum-exp of the split's scaled scores
 *                (ws_lse; -inf and a zero row for an empty split), then
 *                gqa_combine_splits runs on the same stream and writes out.
 *   scale        multiplier of q.k (1/sqrt(D) for standard attention).
 *
 * Returns GQA_OK, or an error code with nothing enqueued.
 */
int gqa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, const int32_t* context_lens, void* out,
                     float* ws_o, float* ws_lse, int B, int Hq, int Hkv, int D, int P,
                     int max_pages, int num_pages, int num_splits, float scale, int dtype,
                     void* stream);

/*
 * Same result as gqa_decode_paged, with the work partition chosen by the library so
 * that unequal context lengths do not leave the GPU idle: the batch's
 * (sequence, KV head, page) items are cut into equal contiguous shares, one per
 * resident wave; a (sequence, KV head) unit cut by a share boundary is finished from
 * its pieces with the log-sum-exp merge of gqa_combine_splits (the NumSplits
 * decomposition of page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", section
 * "核心参数调优：PackGQA与NumSplits的协同舞蹈"). For G >= 16, and for small problems
 * (B * Hkv * max_pages at most 1,024, or 65,536 when G = 1, or 16,384 / 8,192 when G = 2 / 4
 * with at most 4 splits of rows of at least 16 pages; in each case if the split partials fit
 * in the workspace past its counters) it runs the split path with an automatic split count; see
 * gqa_decode_balanced_route. The route depends on the page-table row width max_pages, not
 * on the live lengths: a table sized for a long maximum context always takes the persistent
 * kernel.
 *
 *   workspace        device scratch of at least
 *                    gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D) bytes, 256-byte
 *                    aligned, owned by the caller. Zero it once after allocating it: its
 *                    first GQA_BALANCED_WS_RESERVED bytes are counters that every completed
 *                    call leaves at zero and every call tags with a new epoch (the rest is
 *                    overwritten). One workspace serves
 *                    every shape whose size it covers. Calls that share a workspace must
 *                    not overlap in time and must be enqueued in order (from one host
 *                    thread at a time).
 *   other arguments  as for gqa_decode_paged.
 * Enqueues one kernel on `stream` for G <= 8 (the pieces of units cut by the partition are
 * merged by the piece that finishes last); on the split path the split decode and, with more
 * than one split, the combine.
 */
int gqa_decode_paged_balanced(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* context_lens, void* out,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int D, int P, int max_pages, int num_pages, float scale, int dtype,
                              void* stream);

/* Bytes of the static device buffer of gqa_decode_paged_balanced_noalloc (33.1 MiB per device:
 * the counters plus partial slots for 4096 waves of the largest group, G = 8, D = 128). */
#define GQA_NOALLOC_SCRATCH_BYTES 34701312

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gqa_decode_paged_balanced with the library's own
 * workspace, a file-scope device array of GQA_NOALLOC_SCRATCH_BYTES bytes that each device
 * holds until the process ends. Arguments, result and route are those of
 * gqa_decode_paged_balanced without workspace / workspace_bytes. Nothing is allocated or
 * freed: the first call on a device looks the buffer's address up (hipGetSymbolAddress) and
 * enqueues one small kernel on `stream` that clears its counters; every completed call leaves
 * them zero again. All calls on one device share the buffer, so calls that overlap in time on
 * one device race (enqueue them in order, from one host thread at a time). Returns
 * GQA_ERR_SCRATCH, with nothing enqueued, if a shape needs more than the buffer holds (every
 * supported shape fits: the largest need is GQA_NOALLOC_SCRATCH_BYTES itself).
 */
int gqa_decode_paged_balanced_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* page_table, const int32_t* context_lens,
                                      void* out, int B, int Hq, int Hkv, int D, int P,
                                      int max_pages, int num_pages, float scale, int dtype,
                                      void* stream);

/*
 * One decode step with its own token appended (the per-step KV append: page "TensorRT对
 * Grouped Query Attention的支持进展", section "动态形状与KV Cache管理", the cache grows by
 * one token per generated token). For every sequence b the step's K and V rows
 * k_new[b][kvh][:], v_new[b][kvh][:] are written at position T_b = context_lens[b]
 * (slot T_b % P of page page_table[b][T_b / P], bit copies) and
 * out[b][h] = softmax(scale * q[b][h] . K_b^T) V_b over tokens 0 .. T_b, the new token
 * included (it is read from k_new / v_new, not back from the pool). The pages holding
 * positions 0 .. T_b must be in the page table; pages may be shared between sequences
 * (prefix sharing) except the page that receives the new token. context_lens is not
 * updated (the caller increments it). T_b is clamped to [0, max_pages * P - 1].
 *
 *   q            [B][Hq][D]    dtype
 *   k_new, v_new [B][Hkv][D]   dtype
 *   k_cache,     [num_pages][Hkv][P][D] dtype, written only at the new tokens' slots
 *   v_cache
 *   out          [B][Hq][D]    dtype
 *   workspace    as for gqa_decode_paged_balanced
 * Supported: D in {64, 128}, P = 16, G in {1, 2, 4, 8}, dtype GQA_F32 or GQA_BF16.
 * Enqueues one kernel (decode with the append folded in).
 */
int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                      void* out, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                      int D, int P, int max_pages, int num_pages, float scale, int dtype,
                      void* stream);

/*
 * Decode over an 8-bit floating-point KV pool (the pages quote FP8 KV caches as the next
 * halving of decode bytes: page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", the
 * performance discussion after section "核心参数调优：PackGQA与NumSplits的协同舞蹈"; page
 * "TensorRT对Grouped Query Attention的支持进展", section "显存带宽瓶颈下的理性妥协"). Same
 * result and partition as gqa_decode_paged_balanced with every cache byte x read as
 * k_scale * fp8(x) (K) or v_scale * fp8(x) (V); products and sums in fp32.
 *
 *   q            [B][Hq][D]              bf16
 *   k_cache,     [num_pages][Hkv][P][D]  one byte per element, format kv_dtype
 *   v_cache                              (GQA_FP8_E4M3 or GQA_FP8_E5M2)
 *   k_scale,     per-tensor scales, finite and > 0
 *   v_scale
 *   out          [B][Hq][D]              bf16 (round to nearest even)
 *   workspace    as for gqa_decode_paged_balanced (same size function)
 *   other arguments as for gqa_decode_paged_balanced.
 * Supported: D = 128, G in {1, 2, 4, 8}, P = 16. Enqueues one kernel.
 */
int gqa_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                         float v_scale, const int32_t* page_table, const int32_t* context_lens,
                         void* out, void* workspace, size_t workspace_bytes, int B, int Hq,
                         int Hkv, int D, int P, int max_pages, int num_pages, float scale,
                         int kv_dtype, void* stream);

/*
 * Causal prefill of S new tokens per sequence, with the new K/V appended to
 * the paged cache (page "TensorRT对Grouped Query Attention的支持进展",
 * section "动态形状与KV Cache管理": prefill fills the cache that decode then
 * grows). Causal mask as named in the caption of Figure 2 of page
 * "解锁GQA性能潜力：从批量大小敏感性到高效优化实践": row i (position i of
 * 0..S-1) attends keys 0..i.
 *
 *   q          [B][S][Hq][D]   bf16
 *   k, v       [B][S][Hkv][D]  bf16, the new tokens at positions 0..S-1
 *   k_cache,   [num_pages][Hkv][P][D] bf16; on return (stream order) slot
 *   v_cache    j % P of page page_table[b][j / P] holds k[b][j] / v[b][j]
 *              for every j < S, copied bit for bit; nothing else is written.
 *   page_table [B][max_pages] int32, first ceil(S/P) entries valid per row;
 *              requires max_pages * P >= S. Pages of different sequences
 *              must be distinct.
 *   out        [B][S][Hq][D]   bf16 (round to nearest even)
 */
int gqa_prefill_causal(const void* q, const void* k, const void* v, void* k_cache,
                       void* v_cache, const int32_t* page_table, void* out, int B, int S,
                       int Hq, int Hkv, int D, int P, int max_pages, int num_pages,
                       float scale, int dtype, void* stream);

/*
 * Chunked prefill over an existing paged context. Sequence b already holds past_lens[b]
 * tokens in the pool; this call appends its new_lens[b] <= S new tokens at positions
 * past_lens[b] .. past_lens[b] + new_lens[b] - 1 (page "TensorRT对Grouped Query Attention的
 * 支持进展", section "动态形状与KV Cache管理": the cache grows by the tokens of each step) and
 * computes their attention: new row i, at position past_lens[b] + i, attends keys
 * 0 .. past_lens[b] + i, i.e. every cached token and the new tokens up to itself (the causal
 * mask of the caption of Figure 2 of page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践",
 * aligned to the last key). past_lens = 0, new_lens = S is gqa_prefill_causal.
 *
 *   q          [B][S][Hq][D]   bf16; rows i >= new_lens[b] are ignored
 *   k, v       [B][S][Hkv][D]  bf16, the new tokens (rows i >= new_lens[b] ignored)
 *   k_cache,   [num_pages][Hkv][P][D] bf16; positions < past_lens[b] are read through the
 *   v_cache    page table; on return (stream order) the new rows are in their slots, copied
 *              bit for bit; nothing else is written.
 *   page_table [B][max_pages] int32, the first ceil((past + new) / P) entries valid per row;
 *              pages of different sequences must be distinct.
 *   past_lens, [B] int32 DEVICE arrays. Clamped on the device to 0 <= past <= max_pages*P and
 *   new_lens   0 <= new <= min(S, max_pages*P - past).
 *   out        [B][S][Hq][D]   bf16; rows i < new_lens[b] written, the others untouched.
 * Enqueues two kernels (the append, then the attention reading all K/V from the pool).
 */
int gqa_prefill_paged(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      const int32_t* page_table, const int32_t* past_lens,
                      const int32_t* new_lens, void* out, int B, int S, int Hq, int Hkv, int D,
                      int P, int max_pages, int num_pages, float scale, int dtype, void* stream);

/*
 * Merge split partials, the last step of the NumSplits decomposition (page
 * "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", section
 * "核心参数调优：PackGQA与NumSplits的协同舞蹈": the attention of one query is cut
 * into sub-problems over parts of the context, and their results are combined):
 * M = max_s lse_s, w_s = exp(lse_s - M), out = sum_s w_s o_s / sum_s w_s; a row
 * whose splits are all -inf is zero.
 *   ws_o [B][Hq][num_splits][D] fp32, ws_lse [B][Hq][num_splits] fp32
 *   (natural log), out [B][Hq][D] in out_dtype.
 * Returns GQA_OK, or an error code with nothing enqueued.
 */
int gqa_combine_splits(const float* ws_o, const float* ws_lse, void* out, int B, int Hq, int D,
                       int num_splits, int out_dtype, void* stream);

/* Host-only helpers (no GPU access). */

/* Route gqa_decode_paged_balanced takes for a shape and workspace size: 0 = the persistent
 * balanced kernel (one launch); n >= 1 = the split path with n splits (n > 1 adds the
 * combine). -1 if the arguments are invalid. */
int gqa_decode_balanced_route(int B, int Hq, int Hkv, int D, int max_pages,
                              size_t workspace_bytes);

/* Page ids a call would touch, checked on the host: page_table [B][max_pages] and tokens [B]
 * are HOST arrays; for every b the first ceil(t_b / P) entries of row b, with t_b = tokens[b]
 * clamped to [0, max_pages * P], must lie in [0, num_pages). The token count is what the call
 * reads or writes: context_lens[b] for decode, context_lens[b] + 1 for gqa_decode_append, S
 * for causal prefill, past + new for chunked prefill. Returns GQA_OK or
 * GQA_ERR_INVALID_ARG (also for null arrays or non-positive sizes). Page ids outside the pool
 * are a caller error that the kernels do not check; a library built with GQA_DEBUG defined
 * runs this check in every entry point (after a blocking copy of the table and lengths) and
 * returns its status before enqueueing anything. */
int gqa_check_page_table(const int32_t* page_table, const int32_t* tokens, int B,
                         int max_pages, int P, int num_pages);
size_t gqa_decode_workspace_bytes(int B, int Hq, int D, int num_splits); /* ws_o + ws_lse */
size_t gqa_decode_balanced_workspace_bytes(int B, int Hq, int Hkv, int D);  /* 0 if invalid */
const char* gqa_status_string(int status);
int gqa_validate_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* context_lens, const void* out,
                        const float* ws_o, const float* ws_lse, int B, int Hq, int Hkv, int D,
                        int P, int max_pages, int num_pages, int num_splits, float scale,
                        int dtype);
int gqa_validate_prefill(const void* q, const void* k, const void* v, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const void* out, int B,
                         int S, int Hq, int Hkv, int D, int P, int max_pages, int num_pages,
                         float scale, int dtype);
int gqa_validate_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                            float k_scale, float v_scale, const int32_t* page_table,
                            const int32_t* context_lens, const void* out, int B, int Hq, int Hkv,
                            int D, int P, int max_pages, int num_pages, float scale,
                            int kv_dtype);
int gqa_validate_prefill_paged(const void* q, const void* k, const void* v, const void* k_cache,
                               const void* v_cache, const int32_t* page_table,
                               const int32_t* past_lens, const int32_t* new_lens, const void* out,
                               int B, int S, int Hq, int Hkv, int D, int P, int max_pages,
                               int num_pages, float scale, int dtype);
int gqa_validate_combine(const float* ws_o, const float* ws_lse, const void* out, int B, int Hq,
                         int D, int num_splits, int out_dtype);

/*
 * Test-only: copy the live tokens of a paged cache to a contiguous buffer through
 * the logical -> physical page mapping (page "TensorRT对Grouped Query Attention的支持
 * 进展", section "动态形状与KV Cache管理": the caller passes physical page ids and
 * logical positions are mapped to them; page "TensorRT-LLM与TensorRT核心差异解析",
 * section 4.2.2: a page table maps logically contiguous tokens to scattered
 * fixed-size pages):
 * dst[b][t][kvh][:] = cache[page_table[b][t / P]][kvh][t % P][:] for
 * t < min(context_lens[b], max_pages*P); dst is [B][max_pages*P][Hkv][D] and
 * rows t >= T_b are left untouched. Bit-exact copy of the indexing that the
 * attention kernels use. Returns GQA_OK, or an error code with nothing enqueued.
 */
int gqa_gather_paged(const void* cache, const int32_t* page_table, const int32_t* context_lens,
                     void* dst, int B, int Hkv, int D, int P, int max_pages, int num_pages,
                     int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
