// Balanced paged GQA decode: the whole batch's (sequence, KV head, page) work is cut into
// equal contiguous shares, one per resident wave, so every wave streams the same number
// of pages no matter how unequal the context lengths are.
//
// What is computed is the decode of page "TensorRT-LLM与TensorRT核心差异解析" sections 4.1
// and 4.2.1 through the page table of section 4.2.2 / page "TensorRT对Grouped Query
// Attention的支持进展" section "动态形状与KV Cache管理": out[b][h] = softmax(scale * q K^T) V
// over tokens 0 .. T_b-1, query head h reading KV head h / G. Where a share boundary cuts
// a (sequence, KV head) unit, the pieces are NumSplits-style partials (page
// "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", section
// "核心参数调优：PackGQA与NumSplits的协同舞蹈") merged with the log-sum-exp rule.
//
// Two launches on the caller's stream. Items are ordered b-major, then kv head, then
// page; N items in all, wave w of nw owns [N w / nw, N (w+1) / nw).
//   1. balanced_kernel (persistent): every wave computes N and finds the sequence holding
//      its first item with wave-wide scans of ceil(T_b / P). A unit wholly inside one
//      share is finished and written directly; a cut unit leaves, per piece, a partial
//      (normalised output + natural-log LSE) in the share's slot 0 (its first unit) or
//      slot 1 (its last unit). Each wave keeps two pages in flight in VGPRs while it
//      computes a third; all G <= 8 heads of the group live in the wave, so a K/V row is
//      read once.
//   2. fixup_kernel: one wave per (sequence, KV head) unit merges the pieces of cut units
//      and zero-fills the rows of sequences with T_b = 0. (Merging inside the first
//      kernel would need device-scope fences that write back and invalidate the L2 on
//      every piece: measured slower than this second launch.)
#include "decode_common.h"
#include "decode_mfma.h"

namespace gqa {

constexpr int kBalancedMaxWaves = 4096;  // upper bound of the persistent grid (workspace size)

// Workspace data region: kBalancedMaxWaves x 2 partial slots of G x (D + 1) floats.

// Tokens attended by sequence b: T_b clamped to [0, max_pages * P]; with append = 1 (the
// step's own token is appended at position T_b first) T_b is clamped to
// [0, max_pages * P - 1] and one is added.
__device__ __forceinline__ int seq_len(const int32_t* __restrict__ context_lens, int b,
                                       int max_pages, int append) {
  const int cap = max_pages * kPage - append;
  int T = context_lens[b];
  T = T < 0 ? 0 : (T > cap ? cap : T);
  return T + append;
}
__device__ __forceinline__ int pages_of(const int32_t* __restrict__ context_lens, int b,
                                        int max_pages, int append) {
  return (seq_len(context_lens, b, max_pages, append) + kPage - 1) / kPage;
}

__device__ __forceinline__ long wave_sum(long x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Waves that take a share: all resident waves, or fewer when the batch is small, so that
// a share holds at least kMinShare items (tiny shares cost more in start-up and in pieces
// to merge than they save in parallelism).
constexpr long kMinShare = 4;
__device__ __forceinline__ int active_waves(long N, int resident) {
  const long w = N / kMinShare;
  return w < 1 ? 1 : (w < resident ? (int)w : resident);
}

// share bounds and owner of an item (integer arithmetic shared by writers and mergers)
__device__ __forceinline__ long share_lo(long N, int w, int nw) { return N * w / nw; }
__device__ __forceinline__ int share_owner(long N, long x, int nw) {
  return (int)(((x + 1) * nw - 1) / N);
}

// First sequence b whose items end past item x (so np_b > 0), with np_b and the index of
// its first item: wave-wide inclusive scans of ceil(T_b / P), 64 sequences per step.
// n_first: this lane's page count of the first 64 sequences (already loaded by the caller).
__device__ __forceinline__ void locate_item(const int32_t* __restrict__ context_lens, int B,
                                            int Hkv, int max_pages, int append, long x, int lane,
                                            int n_first, int& b, int& np, long& seq_base) {
  long base = 0;
  for (int c = 0; c < B; c += kWave) {
    const int n = c == 0 ? n_first
                         : (c + lane < B ? pages_of(context_lens, c + lane, max_pages, append) : 0);
    int incl = n;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const unsigned long long hit = __ballot(base + (long)Hkv * incl > x);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      b = uniform(c + L);
      np = uniform(__shfl(n, L));
      seq_base = base + (long)Hkv * (uniform(__shfl(incl, L)) - np);
      return;
    }
    base += (long)Hkv * uniform(__shfl(incl, kWave - 1));
  }
}

// T: q / out element type; TKV: cache element type (T, or an 8-bit float whose per-tensor
// scales are folded in: k_scale into scale_log2, v_scale into out_scale).
template <typename T, int D, int G, typename TKV = T, bool APPEND = false>
__global__ __launch_bounds__(kDecodeThreads) void balanced_kernel(
    const T* __restrict__ q, const TKV* __restrict__ k_cache, const TKV* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, float* __restrict__ slots, int B, int Hq, int Hkv, int max_pages,
    float scale_log2, float out_scale, const TKV* __restrict__ k_new,
    const TKV* __restrict__ v_new, TKV* __restrict__ k_store, TKV* __restrict__ v_store) {
  using S = DecodeShape<TKV, D, G>;
  constexpr int append = APPEND ? 1 : 0;
  static_assert(S::HG == 1, "all heads of the group in one wave");
  constexpr int W32 = S::W32;
  constexpr int E = S::E;
  constexpr int SLOT = G * (D + 1);

  const int lane = lane_id();
  const int r = lane >> 4;
  const int qd = lane & 15;
  const int gw = blockIdx.x * kDecodeWaves + wave_id();

  // ---- total item count N = Hkv * sum_b ceil(T_b / P) ----
  const int n_first = lane < B ? pages_of(context_lens, lane, max_pages, append) : 0;
  long part = n_first;
  for (int bb = lane + kWave; bb < B; bb += kWave)
    part += pages_of(context_lens, bb, max_pages, append);
  const long N = uniform((long)Hkv * wave_sum(part));

  if (N == 0) return;
  const int nw = active_waves(N, gridDim.x * kDecodeWaves);
  if (gw >= nw) return;  // no share: items [N gw / nw, ...) would lie past the last item
  const long lo = share_lo(N, gw, nw);
  const long hi = share_lo(N, gw + 1, nw);
  if (lo >= hi) return;

  // ---- locate the sequence holding item lo ----
  int b = 0, np = 1;
  long seq_base = 0;  // first item of sequence b
  locate_item(context_lens, B, Hkv, max_pages, append, lo, lane, n_first, b, np, seq_base);
  const long rem = lo - seq_base;
  int kvh = (int)(rem / np);
  int pg = (int)(rem % np);
  const size_t page_stride = (size_t)Hkv * S::PAGE;

  // move a cursor to the next item (skipping empty sequences)
  auto advance = [&](int& cb, int& ckv, int& cpg, int& cnp) {
    if (++cpg == cnp) {
      cpg = 0;
      if (++ckv == Hkv) {
        ckv = 0;
        int n = 0;
        do {
          ++cb;
          n = cb < B ? pages_of(context_lens, cb, max_pages, append) : 1;
        } while (n == 0);
        cnp = n;
      }
    }
  };

  // bf16 queries: scores on the matrix core (WaveStateMq, K in its operand layout);
  // fp32: the vector path
  constexpr bool kMq = sizeof(T) == 2;
  using WS = std::conditional_t<kMq, WaveStateMq<T, D, G, TKV>, WaveState<T, D, G, TKV>>;
  const int qsel = kMq ? lane : qd;  // what init() takes
  // page buffers in VGPRs: NB - 1 pages in flight while one is computed (16-bit caches:
  // 4, which leaves one wave per SIMD with D = 128 and measured faster than two waves with
  // 3; 8-bit caches: 3; fp32 with D = 128 and 8 heads: 2, which fits 512 VGPRs)
  constexpr int NB = sizeof(TKV) == 2 ? 4 : (sizeof(TKV) == 4 && D * G >= 1024 ? 2 : 3);
  uint32_t kb[NB][WS::KROWS][WS::KWORDS], vb[NB][4][W32];
  // append: the row of the step's own token (slot (L - 1) % P of the sequence's last page)
  // is read from k_new / v_new instead of the pool (the pool gets it in consume()).
  auto load_page = [&](int buf, int cb, int ckv, int cpg) {
    const size_t page_off = (size_t)page_table[(size_t)cb * max_pages + cpg] * page_stride +
                            (size_t)ckv * S::PAGE;
    const char* kpage = (const char*)k_cache + page_off;
    const char* kp = kpage + r * S::ROW;
    const char* vp = (const char*)v_cache + page_off + r * S::ROW;
    int new_row = -1;
    if constexpr (APPEND) {
      const int L = seq_len(context_lens, cb, max_pages, 1);
      if (cpg == (L - 1) / kPage) new_row = (L - 1) % kPage;
    }
    const size_t new_off = ((size_t)cb * Hkv + ckv) * S::ROW;
    if constexpr (kMq) {
      const int kr = WS::k_row(lane);
      WS::load_k(kr == new_row ? (const char*)k_new + new_off : kpage + kr * S::ROW, lane,
                 kb[buf]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool nr = 4 * i + r == new_row;
      if constexpr (!kMq)
        load_row<TKV, D>(nr ? (const char*)k_new + new_off : kp + i * 4 * S::ROW, qd, kb[buf][i]);
      load_row<TKV, D>(nr ? (const char*)v_new + new_off : vp + i * 4 * S::ROW, qd, vb[buf][i]);
    }
  };

  WS st;
  long seg_start = lo;  // first item of the current segment
  st.init(q + ((size_t)b * Hq + kvh * G) * D, qsel, scale_log2 < 0.f);
  int T_b = seq_len(context_lens, b, max_pages, append);

  auto store_row = [&](T* dst, int hw, float inv) {
    if (r == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float o = st.acc[hw][e] * inv;
        if constexpr (sizeof(T) == 2) {
          ((uint16_t*)dst)[lane_dim<T, D>(qd, e)] = f32_to_bf16(o);
        } else {
          dst[lane_dim<T, D>(qd, e)] = o;
        }
      }
    }
  };

  // Finish the segment that ends at item i: merge the 4 DPP rows, then write the output
  // (the whole unit is in this share) or the piece's partial.
  auto finish = [&](long i) {
    st.merge_rows();
    const long first = i - pg;  // first item of the unit (pg = page of item i)
    if (seg_start == first && pg + 1 == np) {
#pragma unroll
      for (int hw = 0; hw < G; ++hw)
        store_row(out + ((size_t)b * Hq + kvh * G + hw) * D, hw, out_scale / st.l[hw]);
      return;
    }
    const int slot = seg_start == lo ? 0 : 1;
    float* base = slots + ((size_t)gw * 2 + slot) * SLOT;
#pragma unroll
    for (int hw = 0; hw < G; ++hw) {
      const float inv = out_scale / st.l[hw];
      if (r == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) base[hw * (D + 1) + lane_dim<T, D>(qd, e)] = st.acc[hw][e] * inv;
      }
      if (lane == 0) base[hw * (D + 1) + D] = (st.m[hw] + __builtin_log2f(st.l[hw])) * kLn2;
    }
  };

  // Consume item i from buffer `buf`, then move the compute cursor; open a new segment
  // when the next item starts a new unit.
  auto consume = [&](int buf, long i) {
    const int tok0 = pg * kPage + r;
    if (APPEND && pg + 1 == np) {  // write the step's token into its pool slot (once)
      const int slot = (T_b - 1) % kPage;
      const size_t off = (size_t)page_table[(size_t)b * max_pages + pg] * page_stride +
                         (size_t)kvh * S::PAGE + (size_t)slot * S::ROW;
      if constexpr (kMq) {
        if (WS::k_row(lane) == slot) WS::store_k((char*)k_store + off, lane, kb[buf]);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (4 * ii + r == slot) {
          if constexpr (!kMq) store_kv_row<TKV, D>((char*)k_store + off, qd, kb[buf][ii]);
          store_kv_row<TKV, D>((char*)v_store + off, qd, vb[buf][ii]);
        }
      }
    }
    if (pg + 1 < np) {
      st.template page<false>(kb[buf], vb[buf], tok0, T_b, abs_scale(scale_log2));
    } else {
      st.template page<true>(kb[buf], vb[buf], tok0, T_b, abs_scale(scale_log2));
    }
    const bool unit_end = pg + 1 == np;
    if (unit_end || i + 1 == hi) finish(i);
    advance(b, kvh, pg, np);
    if (unit_end && i + 1 < hi) {
      seg_start = i + 1;
      st.init(q + ((size_t)b * Hq + kvh * G) * D, qsel, scale_log2 < 0.f);
      T_b = seq_len(context_lens, b, max_pages, append);
    }
  };

  // The load cursor runs NB - 1 items ahead of the compute cursor (NB page buffers). The
  // prefetch is issued on every step (past the share's end it re-reads the current page,
  // an L2 hit) so that the loads in flight are the same on every path and the wait before
  // each page is exactly "all but the NB - 2 newest pages".
  int lb = b, lkv = kvh, lpg = pg, lnp = np;
  load_page(0, lb, lkv, lpg);
#pragma unroll
  for (int k = 1; k < NB - 1; ++k) {
    if (lo + k < hi) advance(lb, lkv, lpg, lnp);
    load_page(k, lb, lkv, lpg);
  }
  for (long i = lo; i < hi; i += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (i + k + NB - 1 < hi) advance(lb, lkv, lpg, lnp);
      load_page((k + NB - 1) % NB, lb, lkv, lpg);
      consume(k, i + k);
      if (i + k + 1 >= hi) break;
    }
  }
}

// ---- fix-up: merge the pieces of cut units; zero rows of empty sequences ----------------
// One wave per (sequence, KV head, query head of the group). Lane p holds piece p's LSE;
// the weights come from wave reductions; each lane then sums its D / 64 dims over the
// pieces, KB pieces per batch, the first batch's loads issued together with the LSE loads
// (they do not depend on them), so a unit cut into up to KB pieces costs one memory round
// trip after the page-count scan. Pieces are taken 64 at a time.
constexpr int kFixupWaves = 4;

template <typename T, int D, int G>
__global__ __launch_bounds__(kFixupWaves * kWave) void fixup_kernel(
    const float* __restrict__ slots, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, int B, int Hq, int Hkv, int max_pages, int nw, int append) {
  constexpr int SLOT = G * (D + 1);
  constexpr int DL = D / kWave;  // dims per lane
  constexpr int KB = 32;         // pieces per batch
  const int lane = lane_id();
  const long t = (long)blockIdx.x * kFixupWaves + wave_id();
  if (t >= (long)B * Hkv * G) return;
  const long u = t / G;  // (sequence, KV head) unit
  const int hl = (int)(t % G);
  const int b = (int)(u / Hkv);
  const int kvh = (int)(u % Hkv);
  // N and the first item of sequence b in one pass over the page counts
  long part_all = 0, part_before = 0;
  for (int bb = lane; bb < B; bb += kWave) {
    const int n = pages_of(context_lens, bb, max_pages, append);
    part_all += n;
    part_before += bb < b ? n : 0;
  }
  const long N = (long)Hkv * wave_sum(part_all);
  nw = active_waves(N, nw);
  const int np = pages_of(context_lens, b, max_pages, append);
  T* dst = out + ((size_t)b * Hq + kvh * G + hl) * D;
  if (np == 0) {  // T_b == 0: the output is zero
#pragma unroll
    for (int j = 0; j < DL; ++j) {
      if constexpr (sizeof(T) == 2) ((uint16_t*)dst)[lane + kWave * j] = 0;
      else dst[lane + kWave * j] = 0.f;
    }
    return;
  }
  const long first = (long)Hkv * wave_sum(part_before) + (long)kvh * np;
  const int w0 = share_owner(N, first, nw);
  const int w1 = share_owner(N, first + np - 1, nw);
  if (w0 == w1) return;  // finished and written by its wave
  const bool head_is_first = share_lo(N, w0, nw) == first;

  float m_run = -INFINITY, den = 0.f, num[DL];
#pragma unroll
  for (int j = 0; j < DL; ++j) num[j] = 0.f;
  float v[KB][DL];
  for (int c0 = w0; c0 <= w1; c0 += kWave) {
    const int np_c = min(kWave, w1 - c0 + 1);
    // lane p: piece c0 + p (empty shares wrote nothing: weight 0, slot never used)
    const int w = c0 + lane;
    const bool live = lane < np_c && share_lo(N, w, nw) != share_lo(N, w + 1, nw);
    const int slot = (w == w0 && !head_is_first) ? 1 : 0;
    const int off = live ? (int)(((size_t)w * 2 + slot) * SLOT) + hl * (D + 1) : 0;
    const float lse = slots[off + D];
    // data of KB pieces; dead pieces read a valid slot and are replaced by zero
    auto load_batch = [&](int p0) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int p = (p0 + k) & (kWave - 1);
        const int po = __builtin_amdgcn_readlane(off, p);
        const bool pl = p0 + k < np_c && __builtin_amdgcn_readlane((int)live, p) != 0;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
          const float x = slots[po + lane + kWave * j];
          v[k][j] = pl ? x : 0.f;
        }
      }
    };
    load_batch(0);
    float M = live ? lse : -INFINITY;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    M = fmaxf(M, m_run);
    const float rescale = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - M) * kLog2e);
    const float wgt = live ? __builtin_amdgcn_exp2f((lse - M) * kLog2e) : 0.f;
    float ws = wgt;
    for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
    den = den * rescale + ws;
#pragma unroll
    for (int j = 0; j < DL; ++j) num[j] *= rescale;
    m_run = M;
    for (int p0 = 0;;) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float wv = __builtin_amdgcn_readlane(__float_as_int(wgt), (p0 + k) & (kWave - 1));
#pragma unroll
        for (int j = 0; j < DL; ++j) num[j] = fmaf(__int_as_float(wv), v[k][j], num[j]);
      }
      p0 += KB;
      if (p0 >= np_c) break;
      load_batch(p0);
    }
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < DL; ++j) {
    const float o = num[j] * inv;
    const int d = lane + kWave * j;
    if constexpr (sizeof(T) == 2) ((uint16_t*)dst)[d] = f32_to_bf16(o);
    else dst[d] = o;
  }
}

// ---- host side --------------------------------------------------------------------------

template <typename T, int D, int G, typename TKV = T, bool APPEND = false>
static int launch_balanced(const void* q, const void* k, const void* v, const int32_t* pt,
                           const int32_t* lens, void* out, void* slots_ws, int B, int Hq,
                           int Hkv, int max_pages, float scale, hipStream_t s,
                           float out_scale = 1.0f, const void* k_new = nullptr,
                           const void* v_new = nullptr, void* k_store = nullptr,
                           void* v_store = nullptr) {
  // Persistent grid = resident workgroups; a per-device cache of an occupancy query
  // (every thread computes and stores the same value).
  static int grid_cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GQA_ERR_LAUNCH;
  int grid = grid_cache[dev];
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GQA_ERR_LAUNCH;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, balanced_kernel<T, D, G, TKV, APPEND>,
                                                     kDecodeThreads, 0) != hipSuccess)
      return GQA_ERR_LAUNCH;
    grid = cus * (per_cu > 0 ? per_cu : 1);
    if (grid * kDecodeWaves > kBalancedMaxWaves) grid = kBalancedMaxWaves / kDecodeWaves;
    grid_cache[dev] = grid;
  }
  float* slots = (float*)slots_ws;
  hipLaunchKernelGGL((balanced_kernel<T, D, G, TKV, APPEND>), dim3(grid), dim3(kDecodeThreads), 0, s,
                     (const T*)q, (const TKV*)k, (const TKV*)v, pt, lens, (T*)out, slots, B, Hq,
                     Hkv, max_pages, scale * kLog2e, out_scale, (const TKV*)k_new,
                     (const TKV*)v_new, (TKV*)k_store, (TKV*)v_store);
  const unsigned fix_grid = (unsigned)(((long)B * Hq + kFixupWaves - 1) / kFixupWaves);
  hipLaunchKernelGGL((fixup_kernel<T, D, G>), dim3(fix_grid), dim3(kFixupWaves * kWave), 0, s,
                     slots, lens, (T*)out, B, Hq, Hkv, max_pages, grid * kDecodeWaves,
                     APPEND ? 1 : 0);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <typename T, int D>
static int balanced_group(int G, const void* q, const void* k, const void* v, const int32_t* pt,
                          const int32_t* lens, void* out, void* ws, int B, int Hq, int Hkv,
                          int max_pages, float scale, hipStream_t s) {
  switch (G) {
    case 1: return launch_balanced<T, D, 1>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    case 2: return launch_balanced<T, D, 2>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    case 4: return launch_balanced<T, D, 4>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    case 8: return launch_balanced<T, D, 8>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_decode_balanced(const void* q, const void* k, const void* v, const int32_t* pt,
                           const int32_t* lens, void* out, void* ws, int B, int Hq, int Hkv,
                           int D, int max_pages, float scale, int dtype, hipStream_t s) {
  const int G = Hq / Hkv;
  if (dtype == GQA_BF16) {
    if (D == 128) return balanced_group<bf16_t, 128>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    if (D == 64) return balanced_group<bf16_t, 64>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
  } else {
    if (D == 128) return balanced_group<float, 128>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    if (D == 64) return balanced_group<float, 64>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
  }
  return GQA_ERR_UNSUPPORTED;
}

// Decode with the step's own token appended first (k_new / v_new [B][Hkv][D] go to position
// T_b of each sequence, which then attends T_b + 1 tokens); G <= 8.
template <typename T, int D>
static int balanced_group_append(int G, const void* q, const void* k_new, const void* v_new,
                                 void* k, void* v, const int32_t* pt, const int32_t* lens,
                                 void* out, void* ws, int B, int Hq, int Hkv, int max_pages,
                                 float scale, hipStream_t s) {
  switch (G) {
    case 1: return launch_balanced<T, D, 1, T, true>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, 1.0f, k_new, v_new, k, v);
    case 2: return launch_balanced<T, D, 2, T, true>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, 1.0f, k_new, v_new, k, v);
    case 4: return launch_balanced<T, D, 4, T, true>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, 1.0f, k_new, v_new, k, v);
    case 8: return launch_balanced<T, D, 8, T, true>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, 1.0f, k_new, v_new, k, v);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_decode_append(const void* q, const void* k_new, const void* v_new, void* k, void* v,
                         const int32_t* pt, const int32_t* lens, void* out, void* ws, int B,
                         int Hq, int Hkv, int D, int max_pages, float scale, int dtype,
                         hipStream_t s) {
  const int G = Hq / Hkv;
  if (dtype == GQA_BF16) {
    if (D == 128) return balanced_group_append<bf16_t, 128>(G, q, k_new, v_new, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    if (D == 64) return balanced_group_append<bf16_t, 64>(G, q, k_new, v_new, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
  } else {
    if (D == 128) return balanced_group_append<float, 128>(G, q, k_new, v_new, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
    if (D == 64) return balanced_group_append<float, 64>(G, q, k_new, v_new, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s);
  }
  return GQA_ERR_UNSUPPORTED;
}

// 8-bit cache: bf16 q / out, D = 128, G <= 8. k_scale is folded into the score scale and
// v_scale into the output normalisation.
template <typename TKV>
static int balanced_group_fp8(int G, const void* q, const void* k, const void* v,
                              const int32_t* pt, const int32_t* lens, void* out, void* ws, int B,
                              int Hq, int Hkv, int max_pages, float scale, float v_scale,
                              hipStream_t s) {
  switch (G) {
    case 1: return launch_balanced<bf16_t, 128, 1, TKV>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, v_scale);
    case 2: return launch_balanced<bf16_t, 128, 2, TKV>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, v_scale);
    case 4: return launch_balanced<bf16_t, 128, 4, TKV>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, v_scale);
    case 8: return launch_balanced<bf16_t, 128, 8, TKV>(q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages, scale, s, v_scale);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_decode_balanced_fp8(const void* q, const void* k, const void* v, float k_scale,
                               float v_scale, const int32_t* pt, const int32_t* lens, void* out,
                               void* ws, int B, int Hq, int Hkv, int D, int max_pages,
                               float scale, int kv_dtype, hipStream_t s) {
  if (D != 128) return GQA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (kv_dtype == GQA_FP8_E4M3)
    return balanced_group_fp8<fp8e4m3_t>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages,
                                         scale * k_scale, v_scale, s);
  if (kv_dtype == GQA_FP8_E5M2)
    return balanced_group_fp8<fp8e5m2_t>(G, q, k, v, pt, lens, out, ws, B, Hq, Hkv, max_pages,
                                         scale * k_scale, v_scale, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
