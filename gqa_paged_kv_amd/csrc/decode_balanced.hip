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
// One launch on the caller's stream. N items in all, share s of nw is [N s / nw, N (s+1) / nw)
// (nw: the resident waves, fewer for small batches so that a share holds at least kMinShare
// items). 16- and 32-bit caches: items are ordered kv-head-major, then b, then page, nw is a
// multiple of Hkv and wave gw takes share (gw % Hkv) * (nw / Hkv) + gw / Hkv, so share s of
// kv head s / (nw / Hkv) covers the same (b, page) range for every kv head and the waves of a
// workgroup read the same pages of consecutive kv heads, whose blocks lie next to each other
// in the pool, at about the same time. 8-bit caches (two workgroups per compute unit): items
// ordered b-major, then kv head, then page, and wave gw takes share gw. Every wave computes N
// and finds the sequence holding its first item with wave-wide scans of ceil(T_b / P). A
// unit wholly inside one share is finished and written directly; a cut unit leaves, per
// piece, a partial (normalised output + natural-log LSE) in the share's slot 0 (its first
// unit) or slot 1 (its last unit), written with device-coherent write-through stores of
// whole 128-byte lines. After its last page a wave counts its pieces on per-group /
// per-unit counters (device-scope atomics, tagged with the call's epoch); the piece that
// completes a count merges (a group of up to kGroup pieces, then the group partials of a long
// unit) and resets the counter, so no second launch and no cache flush is needed. Each wave keeps pages in
// flight in VGPRs while it computes one; all G <= 8 heads of the group live in the wave,
// so a K/V row is read once. Rows of sequences with T_b = 0 are zero-filled.
#include <atomic>
#include <mutex>

#include "decode_common.h"
#include "decode_mfma.h"

namespace gqa {

#ifndef GQA_DECODE_VALU_SCORES
#define GQA_DECODE_VALU_SCORES 0
#endif

constexpr int kBalancedMaxWaves = 4096;  // upper bound of the persistent grid (workspace size)

// Workspace: GQA_BALANCED_WS_RESERVED bytes of 64-bit counters (kBalancedMaxWaves per-unit
// counters, then 2 kBalancedMaxWaves per-group counters), then kBalancedMaxWaves x 2 partial
// slots of SlotGeom::FLOATS floats (whole 128-byte lines). A counter holds
// (epoch << kEpochShift) + count: every call takes a new, larger epoch from the host, and a
// piece first raises the counter to its call's base (atomic max), then counts on it (atomic
// add), so a partial count that an earlier call left behind (a call that never completed) is
// discarded by the next call. The piece that completes a count resets the counter to zero, so
// a launch replayed with the same epoch (a captured graph) also starts from zero. The
// counters must hold zero (or an earlier epoch's value) before the first call on a workspace.
constexpr int kGroup = 8;  // pieces merged together at the first level
constexpr int kEpochShift = 16;  // counts stay below 2^16 (at most kBalancedMaxWaves pieces)
static_assert(GQA_BALANCED_WS_RESERVED == 3 * kBalancedMaxWaves * 8, "counter region");

// Partial slot of one piece: the G x D normalised output as 16-byte chunks, chunk i * 64 +
// lane holding pair k = 4 i + lane / 16 (head k / JPH, chunk k % JPH of that head's E dims
// of the lane's row-column lane % 16: dims lane_dim(lane % 16, 4 (k % JPH)) .. + 3), then the
// G natural-log LSEs. Every lane of a wave stores and loads 16 contiguous bytes, so each
// wave instruction moves whole 128-byte lines (the stores are write-through, device-coherent).
template <int G, int D>
struct SlotGeom {
  static constexpr int JPH = D / 64;  // 4-float chunks per head per row-column
  static constexpr int NK = G * JPH;  // (head, chunk) pairs per row-column
  static constexpr int NI = (NK + 3) / 4;
  static constexpr int DATA = G * D;
  static constexpr int FLOATS = (G * D + G + 31) / 32 * 32;
};
constexpr int kSc1 = 16;  // cache-policy bit of the buffer builtins: device-scope (sc1)

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float* slots, int G, int D) {
  const int floats = (G * D + G + 31) / 32 * 32;
  return __builtin_amdgcn_make_buffer_rsrc(slots, 0, (int)(kBalancedMaxWaves * 2 * floats * 4),
                                           0x00020000);
}
__device__ __forceinline__ f32x4_t load_sc1(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, kSc1));
}
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, kSc1);
}

// This wave's piece (acc[h] x inv[h], natural-log LSEs lse[h]) into the slot at byte `off`.
// After merge_rows every row of the wave holds the same data, so the four rows store
// different (head, chunk) pairs.
template <int D, int G, typename WS>
__device__ __forceinline__ void store_piece(__amdgpu_buffer_rsrc_t rs, uint32_t off, const WS& st,
                                            const float (&inv)[G], const float (&lse)[G],
                                            int lane) {
  using SG = SlotGeom<G, D>;
  const int r = lane >> 4;
#pragma unroll
  for (int i = 0; i < SG::NI; ++i) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int k = 4 * i + rr;
      if (k < SG::NK && r == rr) {
        const int h = k / SG::JPH, j = k % SG::JPH;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) v[kk] = st.acc[h][4 * j + kk] * inv[h];
      }
    }
    if (4 * i + r < SG::NK) store_sc1(rs, off + (uint32_t)(i * kWave + lane) * 16, v);
  }
  if (lane == 0) {
#pragma unroll
    for (int q4 = 0; q4 < (G + 3) / 4; ++q4) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (4 * q4 + kk < G) v[kk] = lse[4 * q4 + kk];
      store_sc1(rs, off + (uint32_t)(SG::DATA + 4 * q4) * 4, v);
    }
  }
}

// Merge `count` pieces (slot byte offsets off_of(p)) with the log-sum-exp rule. TO_OUT: write
// the G output rows at dst_row (bf16 / fp32); otherwise write a merged partial (same slot
// layout) at byte dst_off. Lane p holds piece p's LSEs; the pieces' data are read KB at a time.
// The first loads of a merge: lane p < min(count, 64) gets piece p's LSEs, every lane its
// part of the data of pieces 0 .. KB - 1 (the last piece repeated past count). Issued ahead of
// the merge itself when two merges run back to back, so that their round trips overlap.
template <int G, int D>
struct MergeFirst {
  static constexpr int KB = 8;
  float lse[G];
  f32x4_t x[KB][SlotGeom<G, D>::NI];
  // Uses every loaded value in an empty asm statement: the loads issued so far stay ahead of
  // this point and are waited for here, together (the scheduler would otherwise move some of
  // them behind the first wait and pay a second round trip).
  __device__ __forceinline__ void ready() {
#pragma unroll
    for (int h = 0; h < G; ++h) asm volatile("" : "+v"(lse[h]));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < SlotGeom<G, D>::NI; ++i) asm volatile("" : "+v"(x[kb][i]));
  }
};
template <int D, int G, typename OffFn>
__device__ __forceinline__ void merge_batch(__amdgpu_buffer_rsrc_t rs, int n_c, int p0,
                                            OffFn off_of, int lane, MergeFirst<G, D>& mf) {
  using SG = SlotGeom<G, D>;
  const int r = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < MergeFirst<G, D>::KB; ++kb) {
    const uint32_t po = off_of(min(p0 + kb, n_c - 1));
#pragma unroll
    for (int i = 0; i < SG::NI; ++i)
      mf.x[kb][i] = 4 * i + r < SG::NK ? load_sc1(rs, po + (uint32_t)(i * kWave + lane) * 16)
                                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}
template <int D, int G, typename OffFn>
__device__ __forceinline__ void merge_first(__amdgpu_buffer_rsrc_t rs, int count, OffFn off_of,
                                            int lane, MergeFirst<G, D>& mf) {
  using SG = SlotGeom<G, D>;
  constexpr int NL = (G + 3) / 4;
  const int n_c = min(kWave, count);
  const uint32_t lo = off_of(lane < n_c ? lane : 0) + SG::DATA * 4;
#pragma unroll
  for (int q4 = 0; q4 < NL; ++q4) {
    const f32x4_t x = load_sc1(rs, lo + 16 * q4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      if (4 * q4 + kk < G) mf.lse[4 * q4 + kk] = x[kk];
  }
  merge_batch<D, G>(rs, n_c, 0, off_of, lane, mf);
}

template <typename T, int D, int G, bool TO_OUT, bool FIRST = false, typename OffFn>
__device__ __forceinline__ void merge_pieces(__amdgpu_buffer_rsrc_t rs, int count, OffFn off_of,
                                             T* __restrict__ dst_row, uint32_t dst_off,
                                             int lane, const MergeFirst<G, D>* first = nullptr) {
  using SG = SlotGeom<G, D>;
  constexpr int NL = (G + 3) / 4;
  constexpr int KB = MergeFirst<G, D>::KB;
  const int r = lane >> 4;
  const int qd = lane & 15;
  float m_run[G], den[G];
  f32x4_t num[SG::NI];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    den[h] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < SG::NI; ++i) num[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the weight of this lane's head in slot chunk i, from per-head values
  auto lane_head_value = [&](const float (&vh)[G], int i) {
    float x = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int k = 4 * i + rr;
      if (k < SG::NK && r == rr) x = vh[k / SG::JPH];
    }
    return x;
  };
  for (int c0 = 0; c0 < count; c0 += kWave) {
    const int n_c = min(kWave, count - c0);
    const bool live = lane < n_c;
    // LSEs and the first batch of pieces' data (issued together: the data does not depend
    // on the LSEs), loaded here or by the caller ahead of time
    auto off_c = [&](int p) { return off_of(c0 + p); };
    MergeFirst<G, D> mf;
    if (FIRST && c0 == 0) {
      mf = *first;
    } else {
      merge_first<D, G>(rs, count - c0, off_c, lane, mf);
      mf.ready();
    }
    const float (&lse)[G] = mf.lse;
    f32x4_t (&x)[KB][SG::NI] = mf.x;
    auto load_batch = [&](int p0) {
      merge_batch<D, G>(rs, n_c, p0, off_c, lane, mf);
      mf.ready();
    };
    float w[G], resc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float M = wave_max_f32(live ? lse[h] : -INFINITY);
      M = fmaxf(M, m_run[h]);
      resc[h] = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run[h] - M) * kLog2e);
      w[h] = live ? __builtin_amdgcn_exp2f((lse[h] - M) * kLog2e) : 0.f;
      const float ws = wave_sum_f32(w[h]);
      den[h] = den[h] * resc[h] + ws;
      m_run[h] = M;
    }
#pragma unroll
    for (int i = 0; i < SG::NI; ++i) num[i] *= lane_head_value(resc, i);
    // Every piece of the batch is accumulated, also those past n_c: their weight (lane
    // p0 + kb >= n_c) is 0 and their data is piece n_c - 1's, so they add 0. Without a branch
    // per piece the compiler keeps every load of the batch ahead of the first wait (one round
    // trip per batch). p0 + kb <= 63, since n_c <= 64 and p0 < n_c is a multiple of KB.
    for (int p0 = 0;;) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float wu[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          wu[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[h]), p0 + kb));
#pragma unroll
        for (int i = 0; i < SG::NI; ++i) num[i] += lane_head_value(wu, i) * x[kb][i];
      }
      p0 += KB;
      if (p0 >= n_c) break;
      load_batch(p0);
    }
  }
  float inv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) inv[h] = 1.0f / den[h];
#pragma unroll
  for (int i = 0; i < SG::NI; ++i) {
    const f32x4_t o = num[i] * lane_head_value(inv, i);
    if constexpr (TO_OUT) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int k = 4 * i + rr;
        if (k < SG::NK && r == rr) {
          T* dst = dst_row + (k / SG::JPH) * D + lane_dim<T, D>(qd, 4 * (k % SG::JPH));
          if constexpr (sizeof(T) == 2) {
            *(u32x2_t*)dst = u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          } else {
            *(f32x4_t*)dst = o;
          }
        }
      }
    } else {
      if (4 * i + r < SG::NK) store_sc1(rs, dst_off + (uint32_t)(i * kWave + lane) * 16, o);
    }
  }
  if constexpr (!TO_OUT) {
    if (lane == 0) {
#pragma unroll
      for (int q4 = 0; q4 < NL; ++q4) {
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          if (4 * q4 + kk < G) v[kk] = m_run[4 * q4 + kk] + __builtin_log2f(den[4 * q4 + kk]) * kLn2;
        store_sc1(rs, dst_off + (uint32_t)(SG::DATA + 4 * q4) * 4, v);
      }
    }
  }
}

// Shape of the Q staging copy where there is none (vector path).
struct NoQStage {
  static constexpr int NPASS = 1, NC = 1;
};

// T: q / out element type; TKV: cache element type (T, or an 8-bit float whose per-tensor
// scales are folded in: k_scale into scale_log2, v_scale into out_scale).
template <typename T, int D, int G, typename TKV = T, bool APPEND = false>
__global__ __launch_bounds__(kDecodeThreads, (is_fp8<TKV>() && G <= 4) ? 2 : 1) void balanced_kernel(
    const T* __restrict__ q, const TKV* __restrict__ k_cache, const TKV* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, float* __restrict__ slots, unsigned long long* __restrict__ counters,
    unsigned long long epoch_base, int B, int Hq, int Hkv, int max_pages, float scale_log2,
    float out_scale, const TKV* __restrict__ k_new,
    const TKV* __restrict__ v_new, TKV* __restrict__ k_store, TKV* __restrict__ v_store) {
  using S = DecodeShape<TKV, D, G>;
  constexpr int append = APPEND ? 1 : 0;
  static_assert(S::HG == 1, "all heads of the group in one wave");
  constexpr int W32 = S::W32;
  constexpr int E = S::E;
  using SG = SlotGeom<G, D>;

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

  if constexpr (!APPEND) {  // T_b = 0: the output rows are zero (one wave per sequence)
    for (int bb = gw; bb < B; bb += (int)gridDim.x * kDecodeWaves) {
      if (pages_of(context_lens, bb, max_pages, 0) != 0) continue;
      T* zrow = out + (size_t)bb * Hq * D;
      for (int x = lane; x < Hq * D; x += kWave) {
        if constexpr (sizeof(T) == 2) ((uint16_t*)zrow)[x] = 0; else zrow[x] = 0.f;
      }
    }
  }
  if (N == 0) return;
  // 16- and 32-bit caches: kv-head-major items (measured faster there; slower for the 8-bit
  // pool, whose kernel runs two workgroups per compute unit)
  constexpr bool kKvMajor = sizeof(TKV) >= 2;
  int nw = active_waves(N, gridDim.x * kDecodeWaves);
  if (kKvMajor && nw >= Hkv) nw -= nw % Hkv;
  if (gw >= nw) return;  // no share: items [N gw / nw, ...) would lie past the last item
  const int sw = kKvMajor && nw >= Hkv ? (gw % Hkv) * (nw / Hkv) + gw / Hkv : gw;  // the share
  const long lo = share_lo(N, sw, nw);
  const long hi = share_lo(N, sw + 1, nw);
  if (lo >= hi) return;

  // ---- locate the kv head and the sequence holding item lo ----
  int b = 0, np = 1, kvh = 0, pg = 0;
  if constexpr (kKvMajor) {
    const long N1 = N / Hkv;  // items of one kv head
    kvh = (int)(lo / N1);
    const long lo1 = lo - (long)kvh * N1;
    long seq_base = 0;  // first item of sequence b within the kv head's items
    locate_item(context_lens, B, 1, max_pages, append, lo1, lane, n_first, b, np, seq_base);
    pg = (int)(lo1 - seq_base);
  } else {
    long seq_base = 0;  // first item of sequence b
    locate_item(context_lens, B, Hkv, max_pages, append, lo, lane, n_first, b, np, seq_base);
    const long rem = lo - seq_base;
    kvh = (int)(rem / np);
    pg = (int)(rem % np);
  }
  const size_t page_stride = (size_t)Hkv * S::PAGE;

  // move a cursor to the next item (skipping empty sequences); kv-head-major: the next page,
  // else the next non-empty sequence, else the first non-empty sequence of the next kv head
  // (past the last item the cursor holds kv head Hkv, which is never read)
  auto advance = [&](int& cb, int& ckv, int& cpg, int& cnp) {
    if (++cpg == cnp) {
      cpg = 0;
      if constexpr (kKvMajor) {
        int n = 0;
        do {
          if (++cb == B) {
            cb = 0;
            if (++ckv == Hkv) {
              n = 1;
              break;
            }
          }
          n = pages_of(context_lens, cb, max_pages, append);
        } while (n == 0);
        cnp = n;
      } else if (++ckv == Hkv) {
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
  // fp32: the vector path. A library built with GQA_DECODE_VALU_SCORES=1 takes the vector
  // path for bf16 too (the same result within rounding; kept to measure the two side by
  // side).
  constexpr bool kMq = sizeof(T) == 2 && !GQA_DECODE_VALU_SCORES;
  using WS = std::conditional_t<kMq, WaveStateMq<T, D, G, TKV>, WaveState<T, D, G, TKV>>;
  const int qsel = kMq ? lane : qd;  // what init() takes
  // 8-bit caches: LDS in which merge_rows rearranges the matrix-core PV (one area per wave)
  constexpr int kStage = (kMq && is_fp8<TKV>()) ? G * D : 4;
  __shared__ __attribute__((aligned(16))) float pv_stage[kDecodeWaves * kStage];
  float* const pv_stage_w = pv_stage + wave_id() * kStage;
  // page buffers in VGPRs: NB - 1 pages in flight while one is computed (16-bit caches:
  // 4, which leaves one wave per SIMD with D = 128 and measured faster than two waves with
  // 3; 8-bit caches: 3; fp32 with D = 128 and 8 heads: 2, which fits 512 VGPRs)
  constexpr int NB = sizeof(TKV) == 2 ? 4 : (sizeof(TKV) == 4 && D * G >= 1024 ? 2 : 3);
  uint32_t kb[NB][WS::KROWS][WS::KWORDS], vb[NB][4][W32];
  // append: the row of the step's own token (slot (L - 1) % P of the sequence's last page)
  // is read from k_new / v_new instead of the pool (the pool gets it in consume()).
  // live = false: a filler load past the share's end (its data is never used), from the
  // first block of the pool, which every such load shares (an L2 hit; re-reading the last
  // page instead would go back to HBM, since the streaming hint does not keep it in L2).
  auto load_page = [&](int buf, int cb, int ckv, int cpg, bool live) {
    const size_t page_off =
        live ? (size_t)page_table[(size_t)cb * max_pages + cpg] * page_stride +
                   (size_t)ckv * S::PAGE
             : 0;
    const char* kpage = (const char*)k_cache + page_off;
    const char* kp = kpage + r * S::ROW;
    const char* vp = (const char*)v_cache + page_off + r * S::ROW;
    int new_row = -1;
    if constexpr (APPEND) {
      const int L = seq_len(context_lens, cb, max_pages, 1);
      if (live && cpg == (L - 1) / kPage) new_row = (L - 1) % kPage;
    }
    const size_t new_off = ((size_t)cb * Hkv + ckv) * S::ROW;
    if constexpr (kMq) {
      const int kr = WS::k_row(lane);
      WS::load_k(kr == new_row ? (const char*)k_new + new_off : kpage + kr * S::ROW, lane,
                 kb[buf]);
    }
    if constexpr (kMq && is_fp8<TKV>() && !APPEND) {
      // 8-bit V rows by 16-byte streaming loads: lanes 2m and 2m + 1 of a row group together
      // need dims 16m .. 16m + 15 of rows r, r + 4, r + 8, r + 12; the even lane reads rows
      // r and r + 8, the odd lane rows r + 4 and r + 12 (raw words, rearranged in page()).
      const char* vpage = (const char*)v_cache + page_off;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = r + 4 * ((qd & 1) + 2 * c);
        const u32x4_t x = __builtin_nontemporal_load(
            (const u32x4_t*)(vpage + row * S::ROW + 16 * (qd >> 1)));
        vb[buf][2 * c][0] = x[0];
        vb[buf][2 * c][1] = x[1];
        vb[buf][2 * c + 1][0] = x[2];
        vb[buf][2 * c + 1][1] = x[3];
      }
    } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool nr = 4 * i + r == new_row;
      if constexpr (!kMq)
        load_row_nt<TKV, D>(nr ? (const char*)k_new + new_off : kp + i * 4 * S::ROW, qd, kb[buf][i]);
      load_row_nt<TKV, D>(nr ? (const char*)v_new + new_off : vp + i * 4 * S::ROW, qd, vb[buf][i]);
    }
    }
  };

  WS st;
  long seg_start = lo;  // first item of the current segment
  st.init(q + ((size_t)b * Hq + kvh * G) * D, qsel, scale_log2 < 0.f);
  // Matrix-core path: the Q words of the unit the load cursor entered last, fetched when it
  // enters it (NB - 1 items ahead of the compute cursor), so that opening a segment does not
  // wait on a Q load issued behind the pages in flight. qn_unit: that unit (b * Hkv + kv
  // head), or -1.
  using QS = std::conditional_t<kMq, WS, NoQStage>;
  u32x4_t qn[QS::NPASS][QS::NC];
  long qn_unit = -1;
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

  // Pieces of cut units held by this share (at most one per slot), published at its end.
  struct Piece {
    long first;  // first item of the unit
    int np;      // the unit's item count
    int valid;
    size_t dst;  // output row offset of the unit
  };
  Piece piece0{0, 0, 0, 0}, piece1{0, 0, 0, 0};
  const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slots, G, D);
  auto slot_off = [&](int w, int sl) {
    return (uint32_t)(((size_t)w * 2 + sl) * SG::FLOATS * 4);
  };

  // Finish the segment that ends at item i: merge the 4 DPP rows, then write the output
  // (the whole unit is in this share) or the piece's partial (write-through stores).
  auto finish = [&](long i) {
    if constexpr (kMq) st.merge_rows(pv_stage_w); else st.merge_rows();
    const long first = i - pg;  // first item of the unit (pg = page of item i)
    if (seg_start == first && pg + 1 == np) {
#pragma unroll
      for (int hw = 0; hw < G; ++hw)
        store_row(out + ((size_t)b * Hq + kvh * G + hw) * D, hw, out_scale / st.l[hw]);
      return;
    }
    const int slot = seg_start == lo ? 0 : 1;
    float inv[G], lse[G];
#pragma unroll
    for (int hw = 0; hw < G; ++hw) {
      inv[hw] = out_scale / st.l[hw];
      lse[hw] = (st.m[hw] + __builtin_log2f(st.l[hw])) * kLn2;
    }
    store_piece<D, G>(rs, slot_off(sw, slot), st, inv, lse, lane);
    const Piece pc{uniform(first), uniform(np), 1,
                   (size_t)uniform((long)(((size_t)b * Hq + kvh * G) * D))};
    if (slot == 0) piece0 = pc; else piece1 = pc;
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
      if constexpr (kMq) {
        if (qn_unit == (long)b * Hkv + kvh) {
          st.init_from(qn);
        } else {
          st.init(q + ((size_t)b * Hq + kvh * G) * D, qsel, scale_log2 < 0.f);
        }
      } else {
        st.init(q + ((size_t)b * Hq + kvh * G) * D, qsel, scale_log2 < 0.f);
      }
      T_b = seq_len(context_lens, b, max_pages, append);
    }
  };

  // The load cursor runs NB - 1 items ahead of the compute cursor (NB page buffers). The
  // prefetch is issued on every step (past the share's end as a filler load, see load_page)
  // so that the loads in flight are the same on every path and the wait before each page
  // is exactly "all but the NB - 2 newest pages".
  int lb = b, lkv = kvh, lpg = pg, lnp = np;
  auto advance_load = [&]() {
    advance(lb, lkv, lpg, lnp);
    if constexpr (kMq) {
      if (lpg == 0) {  // the load cursor entered a new unit
        WS::fetch_q(q + ((size_t)lb * Hq + lkv * G) * D, lane, scale_log2 < 0.f, qn);
        qn_unit = (long)lb * Hkv + lkv;
      }
    }
  };
  load_page(0, lb, lkv, lpg, true);
#pragma unroll
  for (int k = 1; k < NB - 1; ++k) {
    const bool live = lo + k < hi;
    if (live) advance_load();
    load_page(k, lb, lkv, lpg, live);
  }
  for (long i = lo; i < hi; i += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const bool live = i + k + NB - 1 < hi;
      if (live) advance_load();
      load_page((k + NB - 1) % NB, lb, lkv, lpg, live);
      consume(k, i + k);
      if (i + k + 1 >= hi) break;
    }
  }

  // Publish the pieces. The wait covers this wave's partial stores; only then is a piece
  // counted. Units of up to kGroup pieces: the piece that completes its group's count
  // merges the unit into the output. Longer units: the last piece of each group of kGroup
  // consecutive pieces merges the group into a partial (in the group's first slot) and
  // counts it on the unit's counter; the last group merges the group partials.
  if ((piece0.valid | piece1.valid) == 0) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  unsigned long long* const unit_cnt = counters;
  unsigned long long* const group_cnt = counters + kBalancedMaxWaves;
  // This piece's arrival number on counter c within this call (1 = first). Both atomics act
  // on one address from one lane, so they take effect in program order (the language's
  // coherence rule for one object).
  auto count_in = [&](unsigned long long* c) {
    unsigned long long old = 0;
    if (lane == 0) {
      __hip_atomic_fetch_max(c, epoch_base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old = (unsigned long long)uniform((long)old);
    asm volatile("" ::: "memory");
    return (long)(old + 1 - epoch_base);
  };
  // The piece that completes a count sets the counter back to zero, which every later call
  // (a new epoch, or a replay of this same launch with the same epoch) starts from.
  auto clear = [&](unsigned long long* c) {
    if (lane == 0) __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // The group counter of a piece and the shape of its unit's merge.
  struct Plan {
    int w0, s0, g, gfirst, gsize, ngroups;
    unsigned long long* gc;
  };
  auto plan_of = [&](const Piece& pc) {
    Plan pl;
    pl.w0 = share_owner(N, pc.first, nw);
    const int w1 = share_owner(N, pc.first + pc.np - 1, nw);
    const int npc = w1 - pl.w0 + 1;                                   // pieces of the unit
    pl.s0 = share_lo(N, pl.w0, nw) == pc.first ? 0 : 1;               // slot of piece 0
    pl.g = (sw - pl.w0) / kGroup;
    pl.gfirst = pl.w0 + pl.g * kGroup;
    pl.gsize = min(kGroup, npc - pl.g * kGroup);
    pl.ngroups = (npc + kGroup - 1) / kGroup;
    pl.gc = group_cnt + 2 * pl.gfirst + (pl.g == 0 ? pl.s0 : 0);
    return pl;
  };
  auto piece_off_of = [&](const Plan& pl) {
    return [=](int p) { return slot_off(pl.gfirst + p, (pl.g == 0 && p == 0) ? pl.s0 : 0); };
  };
  // The rest of a piece's publication once it has completed its group's count.
  // (A counter is reset after the merge it released: the reset is a write-through store, and
  // a store issued before the merge's loads would have its acknowledgement waited for first.)
  auto complete = [&](const Piece& pc, const Plan& pl) {
    const auto piece_off = piece_off_of(pl);
    if (pl.ngroups == 1) {
      merge_pieces<T, D, G, true>(rs, pl.gsize, piece_off, out + pc.dst, 0u, lane);
      clear(pl.gc);
      return;
    }
    merge_pieces<T, D, G, false>(rs, pl.gsize, piece_off, out, piece_off(0), lane);
    clear(pl.gc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    unsigned long long* uc = unit_cnt + pl.w0;
    if (count_in(uc) != pl.ngroups) return;
    auto group_off = [&](int gg) { return slot_off(pl.w0 + gg * kGroup, gg == 0 ? pl.s0 : 0); };
    merge_pieces<T, D, G, true>(rs, pl.ngroups, group_off, out + pc.dst, 0u, lane);
    clear(uc);
  };
  // Both pieces are counted before either is merged, so that the two counters' round trips
  // overlap; when this wave completes both units (each a single group of pieces), the first
  // loads of the two merges are issued together as well.
  const Plan p0 = piece0.valid ? plan_of(piece0) : Plan{};
  const Plan p1 = piece1.valid ? plan_of(piece1) : Plan{};
  unsigned long long old0 = 0, old1 = 0;
  if (lane == 0) {
    if (piece0.valid) {
      __hip_atomic_fetch_max(p0.gc, epoch_base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old0 = __hip_atomic_fetch_add(p0.gc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (piece1.valid) {
      __hip_atomic_fetch_max(p1.gc, epoch_base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old1 = __hip_atomic_fetch_add(p1.gc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const bool done0 = piece0.valid && uniform((long)old0) + 1 - (long)epoch_base == p0.gsize;
  const bool done1 = piece1.valid && uniform((long)old1) + 1 - (long)epoch_base == p1.gsize;
  asm volatile("" ::: "memory");
  if constexpr (G <= 4) {
    if (done0 && done1 && p0.ngroups == 1 && p1.ngroups == 1) {
      const auto off0 = piece_off_of(p0);
      const auto off1 = piece_off_of(p1);
      MergeFirst<G, D> f0, f1;
      merge_first<D, G>(rs, p0.gsize, off0, lane, f0);
      merge_first<D, G>(rs, p1.gsize, off1, lane, f1);
      f0.ready();
      f1.ready();
      merge_pieces<T, D, G, true, true>(rs, p0.gsize, off0, out + piece0.dst, 0u, lane, &f0);
      merge_pieces<T, D, G, true, true>(rs, p1.gsize, off1, out + piece1.dst, 0u, lane, &f1);
      clear(p0.gc);
      clear(p1.gc);
      return;
    }
  }
  if (done0) complete(piece0, p0);
  if (done1) complete(piece1, p1);
}

// ---- static scratch of the allocation-free entry point -----------------------------------

// One balanced-decode workspace per device in a file-scope device array: counters, then the
// partial slots for the largest supported group (G = 8, D = 128); the split route's partials
// fit in the slot area for every supported shape. Every call on a device shares it.
static_assert(GQA_NOALLOC_SCRATCH_BYTES ==
                  GQA_BALANCED_WS_RESERVED + (size_t)kBalancedMaxWaves * 2 *
                                                 SlotGeom<8, 128>::FLOATS * sizeof(float),
              "static scratch size");
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

__global__ void zero_words(unsigned long long* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// Device address of this device's `scratch`, looked up once per device (with the device
// current) by hipGetSymbolAddress; on that first call the counter region is cleared by a small
// kernel on `s`. Host code never uses the array's own name, which is a host-side stand-in.
int noalloc_scratch(void** ptr, hipStream_t s) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_LAUNCH;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
        return GQA_ERR_LAUNCH;
      hipLaunchKernelGGL(zero_words, dim3(48), dim3(256), 0, s, (unsigned long long*)q,
                         (int)(GQA_BALANCED_WS_RESERVED / 8));
      if (hipGetLastError() != hipSuccess) return GQA_ERR_LAUNCH;
      addr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *ptr = p;
  return GQA_OK;
}

// ---- host side --------------------------------------------------------------------------

// Epoch of the next call, shifted into place: a process-wide count of launches of the
// balanced kernel, so every call on a workspace sees a larger epoch than the calls enqueued
// before it (calls that share a workspace are enqueued in order from one thread at a time).
static unsigned long long next_epoch_base() {
  static std::atomic<unsigned long long> epoch{0};
  return (epoch.fetch_add(1, std::memory_order_relaxed) + 1) << kEpochShift;
}

template <typename T, int D, int G, typename TKV = T, bool APPEND = false>
static int launch_balanced(const void* q, const void* k, const void* v, const int32_t* pt,
                           const int32_t* lens, void* out, void* slots_ws, int B, int Hq,
                           int Hkv, int max_pages, float scale, hipStream_t s,
                           float out_scale = 1.0f, const void* k_new = nullptr,
                           const void* v_new = nullptr, void* k_store = nullptr,
                           void* v_store = nullptr) {
  // Persistent grid = resident workgroups; a per-device cache of an occupancy query
  // (threads that race on a first call all compute and store the same value).
  static std::atomic<int> grid_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GQA_ERR_LAUNCH;
  int grid = grid_cache[dev].load(std::memory_order_relaxed);
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GQA_ERR_LAUNCH;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, balanced_kernel<T, D, G, TKV, APPEND>,
                                                     kDecodeThreads, 0) != hipSuccess)
      return GQA_ERR_LAUNCH;
    grid = cus * (per_cu > 0 ? per_cu : 1);
    if (grid * kDecodeWaves > kBalancedMaxWaves) grid = kBalancedMaxWaves / kDecodeWaves;
    grid_cache[dev].store(grid, std::memory_order_relaxed);
  }
  unsigned long long* counters = (unsigned long long*)slots_ws;
  float* slots = (float*)((char*)slots_ws + GQA_BALANCED_WS_RESERVED);
  hipLaunchKernelGGL((balanced_kernel<T, D, G, TKV, APPEND>), dim3(grid), dim3(kDecodeThreads), 0, s,
                     (const T*)q, (const TKV*)k, (const TKV*)v, pt, lens, (T*)out, slots, counters,
                     next_epoch_base(), B, Hq, Hkv, max_pages, scale * kLog2e, out_scale,
                     (const TKV*)k_new,
                     (const TKV*)v_new, (TKV*)k_store, (TKV*)v_store);
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
