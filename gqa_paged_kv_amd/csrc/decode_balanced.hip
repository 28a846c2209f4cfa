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
// Three launches on the caller's stream:
//   1. prefix_kernel   np_b = ceil(T_b / P) and its exclusive prefix sum over b;
//   2. stream_kernel   persistent: wave w owns items [N w / W, N (w+1) / W) of the
//                      b-major, then kv-head, then page ordered item list (N items).
//                      A unit wholly inside one share is finished and written directly;
//                      a cut unit leaves a partial (normalised output + natural-log LSE)
//                      in the share's slot 0 (its first unit) or slot 1 (its last unit);
//   3. fixup_kernel    merges the partials of every cut unit and zero-fills T_b = 0 rows.
// Each wave keeps the next page in flight in VGPRs while computing the current one;
// all G <= 8 heads of the group live in the wave, so a K/V row is read once.
#include "decode_common.h"

namespace gqa {

constexpr int kBalancedMaxWaves = 4096;  // upper bound of the persistent grid (workspace size)

// Bytes of the workspace: [slots: waves x 2 x G x (D + 1) floats][prefix: B + 1 ints].
static size_t balanced_slot_floats(int G, int D) { return (size_t)kBalancedMaxWaves * 2 * G * (D + 1); }

// ---- 1. page counts and their prefix sum (one workgroup of 256 threads) ---------------
__device__ __forceinline__ int pages_of(const int32_t* __restrict__ context_lens, int b,
                                        int max_pages) {
  int T = context_lens[b];
  T = T < 0 ? 0 : (T > max_pages * kPage ? max_pages * kPage : T);
  return (T + kPage - 1) / kPage;
}

__global__ __launch_bounds__(256) void prefix_kernel(const int32_t* __restrict__ context_lens,
                                                     int32_t* __restrict__ prefix, int B,
                                                     int max_pages) {
  __shared__ int wave_tot[4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int per = (B + 255) / 256;  // consecutive sequences per thread
  const int b0 = min(t * per, B), b1 = min(b0 + per, B);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += pages_of(context_lens, b, max_pages);
  int incl = sum;  // inclusive scan inside the wave
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_tot[t >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (t >> 6); ++w) base += wave_tot[w];
  int run = base + incl - sum;  // exclusive prefix of this thread's first sequence
  for (int b = b0; b < b1; ++b) {
    prefix[b] = run;
    run += pages_of(context_lens, b, max_pages);
  }
  if (t == 255) prefix[B] = run;
}

// Largest b in [0, B) with Hkv * prefix[b] <= x, for 0 <= x < Hkv * prefix[B] (then
// np_b > 0). 64-way search: every step samples 64 prefix entries, one per lane.
__device__ __forceinline__ int find_sequence(const int32_t* __restrict__ prefix, int B, int Hkv,
                                             long x, int lane) {
  int lo = 0, hi = B;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool le = idx < hi && (long)Hkv * prefix[idx] <= x;
    const int cnt = __popcll(__ballot(le));  // lanes 0 .. cnt-1 (lane 0 always)
    const int nlo = lo + (cnt - 1) * step;
    hi = min(hi, lo + cnt * step);
    lo = nlo;
  }
  return lo;
}

// ---- 2. persistent streaming decode (G <= 8) --------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void stream_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ prefix, T* __restrict__ out, float* __restrict__ slots, int B,
    int Hq, int Hkv, int max_pages, float scale_log2) {
  using S = DecodeShape<T, D, G>;
  static_assert(S::HG == 1, "all heads of the group in one wave");
  constexpr int W32 = S::W32;
  constexpr int E = S::E;

  const int lane = lane_id();
  const int r = lane >> 4;
  const int qd = lane & 15;
  const int nw = gridDim.x * kDecodeWaves;
  const int gw = blockIdx.x * kDecodeWaves + wave_id();
  const long N = (long)Hkv * prefix[B];
  const long lo = N * gw / nw;
  const long hi = N * (gw + 1) / nw;
  if (lo >= hi) return;

  // cursor over items: sequence b, kv head kvh, page pg of np pages
  int b = find_sequence(prefix, B, Hkv, lo, lane);
  int np = prefix[b + 1] - prefix[b];
  long rem = lo - (long)Hkv * prefix[b];
  int kvh = (int)(rem / np);
  int pg = (int)(rem % np);
  const size_t page_stride = (size_t)Hkv * S::PAGE;

  auto advance = [&](int& cb, int& ckv, int& cpg, int& cnp) {
    if (++cpg == cnp) {
      cpg = 0;
      if (++ckv == Hkv) {
        ckv = 0;
        do {
          ++cb;
        } while (cb < B && prefix[cb + 1] == prefix[cb]);
        cnp = cb < B ? prefix[cb + 1] - prefix[cb] : 1;
      }
    }
  };

  uint32_t kb[2][4][W32], vb[2][4][W32];
  auto load_page = [&](int buf, int cb, int ckv, int cpg) {
    const size_t off = (size_t)page_table[(size_t)cb * max_pages + cpg] * page_stride +
                       (size_t)ckv * S::PAGE + r * S::ROW;
    const char* kp = (const char*)k_cache + off;
    const char* vp = (const char*)v_cache + off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_row<T, D>(kp + i * 4 * S::ROW, qd, kb[buf][i]);
      load_row<T, D>(vp + i * 4 * S::ROW, qd, vb[buf][i]);
    }
  };

  WaveState<T, D, G> st;
  long seg_start = lo;  // first item of the current segment
  int seg_pg0 = pg;     // its page within the unit
  st.init(q + ((size_t)b * Hq + kvh * G) * D, qd);
  int T_b = min(context_lens[b], max_pages * kPage);

  // Finish the segment that ends at the current item: merge rows, then write the final
  // output (the whole unit is in this share) or a partial into slot 0 / 1.
  auto finish = [&](bool whole_unit) {
    st.merge_rows();
    if (whole_unit) {
#pragma unroll
      for (int hw = 0; hw < G; ++hw) {
        const float inv = 1.0f / st.l[hw];
        T* dst = out + ((size_t)b * Hq + kvh * G + hw) * D;
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
      }
    } else {
      const int slot = seg_start == lo ? 0 : 1;
      float* base = slots + ((size_t)gw * 2 + slot) * G * (D + 1);
#pragma unroll
      for (int hw = 0; hw < G; ++hw) {
        const float inv = 1.0f / st.l[hw];
        if (r == 0) {
#pragma unroll
          for (int e = 0; e < E; ++e) base[hw * (D + 1) + lane_dim<T, D>(qd, e)] = st.acc[hw][e] * inv;
        }
        if (lane == 0) base[hw * (D + 1) + D] = (st.m[hw] + __builtin_log2f(st.l[hw])) * kLn2;
      }
    }
  };

  // Consume item i (the current cursor) from buffer `buf`, then open the next segment if
  // the next item starts a new unit.
  auto consume = [&](int buf, long i) {
    const int tok0 = pg * kPage + r;
    if (pg + 1 < np) {
      st.template page<false>(kb[buf], vb[buf], tok0, T_b, scale_log2);
    } else {
      st.template page<true>(kb[buf], vb[buf], tok0, T_b, scale_log2);
    }
    const bool unit_end = pg + 1 == np;
    if (unit_end || i + 1 == hi) {
      finish(unit_end && seg_pg0 == 0);
    }
    advance(b, kvh, pg, np);
    if (unit_end && i + 1 < hi) {
      seg_start = i + 1;
      seg_pg0 = 0;
      st.reset();
      st.init(q + ((size_t)b * Hq + kvh * G) * D, qd);
      T_b = min(context_lens[b], max_pages * kPage);
    }
  };

  // The load cursor runs one item ahead of the compute cursor. The prefetch is issued on
  // every step (past the share's end it re-reads the current page, an L2 hit) so that the
  // number of loads in flight is the same on every path and the wait before each page is
  // exactly "all but the newest page".
  int lb = b, lkv = kvh, lpg = pg, lnp = np;
  load_page(0, lb, lkv, lpg);
  for (long i = lo; i < hi; i += 2) {
    if (i + 1 < hi) advance(lb, lkv, lpg, lnp);
    load_page(1, lb, lkv, lpg);
    consume(0, i);
    if (i + 1 >= hi) break;
    if (i + 2 < hi) advance(lb, lkv, lpg, lnp);
    load_page(0, lb, lkv, lpg);
    consume(1, i + 1);
  }
}

// ---- 3. merge the partials of cut units; zero rows of empty sequences --------------------
// One workgroup per (sequence, KV head) unit. The pieces' LSEs are read once, in parallel,
// into LDS and turned into normalised weights; each output then sums independent loads.
constexpr int kFixupThreads = 256;
constexpr int kFixupMaxParts = 512;  // pieces merged per LDS pass

template <typename T, int D, int G>
__global__ __launch_bounds__(kFixupThreads) void fixup_kernel(const float* __restrict__ slots,
                                                             const int32_t* __restrict__ prefix,
                                                             T* __restrict__ out, int B, int Hq,
                                                             int Hkv, int nw) {
  __shared__ float wgt[kFixupMaxParts * G];
  __shared__ int part_off[kFixupMaxParts];  // float offset of each piece's slot
  __shared__ float red_m[G], red_l[G];
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int kvh = u % Hkv;
  const int np = prefix[b + 1] - prefix[b];
  const long N = (long)Hkv * prefix[B];
  T* dst = out + ((size_t)b * Hq + kvh * G) * D;
  if (np == 0) {  // T_b == 0: the output is zero
    for (int i = threadIdx.x; i < G * D; i += kFixupThreads) {
      if constexpr (sizeof(T) == 2) ((uint16_t*)dst)[i] = 0; else dst[i] = 0.f;
    }
    return;
  }
  const long first = (long)Hkv * prefix[b] + (long)kvh * np;
  const long last = first + np - 1;
  // wave w owns [N w / nw, N (w+1) / nw): the owner of item x is floor(((x+1) nw - 1) / N)
  const int w0 = (int)(((first + 1) * nw - 1) / N);
  const int w1 = (int)(((last + 1) * nw - 1) / N);
  if (w0 == w1) return;  // finished and written by its wave
  const bool head_is_first = (N * w0 / nw) == first;

  float acc[(G * D + kFixupThreads - 1) / kFixupThreads];
  for (int k = 0; k < (G * D + kFixupThreads - 1) / kFixupThreads; ++k) acc[k] = 0.f;
  float m_run[G], l_run[G];  // running max / sum per head (same in every thread)
  for (int hl = 0; hl < G; ++hl) { m_run[hl] = -INFINITY; l_run[hl] = 0.f; }

  for (int c0 = w0; c0 <= w1; c0 += kFixupMaxParts) {
    const int nparts = min(kFixupMaxParts, w1 - c0 + 1);
    // piece p = wave c0 + p; empty shares (fewer items than waves) wrote nothing
    for (int i = threadIdx.x; i < nparts * G; i += kFixupThreads) {
      const int p = i / G, hl = i % G;
      const int w = c0 + p;
      const int slot = (w == w0 && !head_is_first) ? 1 : 0;
      const size_t off = (((size_t)w * 2 + slot) * G + hl) * (D + 1);
      const bool empty = N * w / nw == N * (w + 1) / nw;
      wgt[i] = empty ? -INFINITY : slots[off + D];
      if (hl == 0) part_off[p] = (int)(((size_t)w * 2 + slot) * G * (D + 1));
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int hl = threadIdx.x;
      float M = m_run[hl];
      for (int p = 0; p < nparts; ++p) M = fmaxf(M, wgt[p * G + hl]);
      red_m[hl] = M;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nparts * G; i += kFixupThreads) {
      const float lse = wgt[i];
      wgt[i] = lse == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lse - red_m[i % G]) * kLog2e);
    }
    __syncthreads();
    for (int k = 0; k * kFixupThreads + (int)threadIdx.x < G * D; ++k) {
      const int idx = k * kFixupThreads + threadIdx.x;
      const int hl = idx / D, d = idx % D;
      const float scale_old = m_run[hl] == -INFINITY ? 0.f
                              : __builtin_amdgcn_exp2f((m_run[hl] - red_m[hl]) * kLog2e);
      float a = acc[k] * scale_old;
#pragma unroll 4
      for (int p = 0; p < nparts; ++p) {
        const float wv = wgt[p * G + hl];  // 0 for an empty share: its slot was never written
        if (wv != 0.f) a = fmaf(wv, slots[part_off[p] + hl * (D + 1) + d], a);
      }
      acc[k] = a;
    }
    for (int hl = 0; hl < G; ++hl) {
      const float scale_old = m_run[hl] == -INFINITY ? 0.f
                              : __builtin_amdgcn_exp2f((m_run[hl] - red_m[hl]) * kLog2e);
      float l = l_run[hl] * scale_old;
      for (int p = 0; p < nparts; ++p) l += wgt[p * G + hl];
      l_run[hl] = l;
      m_run[hl] = red_m[hl];
    }
    __syncthreads();
  }
  for (int k = 0; k * kFixupThreads + (int)threadIdx.x < G * D; ++k) {
    const int idx = k * kFixupThreads + threadIdx.x;
    const float o = acc[k] / l_run[idx / D];
    if constexpr (sizeof(T) == 2) ((uint16_t*)dst)[idx] = f32_to_bf16(o); else dst[idx] = o;
  }
}

// ---- host side --------------------------------------------------------------------------

template <typename T, int D, int G>
static int launch_balanced(const void* q, const void* k, const void* v, const int32_t* pt,
                           const int32_t* lens, void* out, void* workspace, int B, int Hq,
                           int Hkv, int max_pages, float scale, hipStream_t s) {
  static int grid_cache[64] = {0};  // persistent grid per device (resident workgroups)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GQA_ERR_LAUNCH;
  int grid = grid_cache[dev];
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GQA_ERR_LAUNCH;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<T, D, G>,
                                                     kDecodeThreads, 0) != hipSuccess)
      return GQA_ERR_LAUNCH;
    grid = cus * (per_cu > 0 ? per_cu : 1);
    if (grid * kDecodeWaves > kBalancedMaxWaves) grid = kBalancedMaxWaves / kDecodeWaves;
    grid_cache[dev] = grid;
  }
  float* slots = (float*)workspace;
  int32_t* prefix = (int32_t*)(slots + balanced_slot_floats(G, D));
  hipLaunchKernelGGL(prefix_kernel, dim3(1), dim3(256), 0, s, lens, prefix, B, max_pages);
  hipLaunchKernelGGL((stream_kernel<T, D, G>), dim3(grid), dim3(kDecodeThreads), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, pt, lens, prefix, (T*)out, slots, B,
                     Hq, Hkv, max_pages, scale * kLog2e);
  hipLaunchKernelGGL((fixup_kernel<T, D, G>), dim3((unsigned)(B * Hkv)), dim3(kFixupThreads), 0, s,
                     slots, prefix, (T*)out, B, Hq, Hkv, grid * kDecodeWaves);
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

size_t balanced_workspace_bytes(int B, int Hq, int Hkv, int D) {
  const int G = Hq / Hkv;
  return balanced_slot_floats(G, D) * sizeof(float) + (size_t)(B + 1) * sizeof(int32_t);
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

}  // namespace gqa
