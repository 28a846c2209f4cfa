// Paged GQA decode on gfx950: one workgroup (4 waves) per (sequence b, KV head kvh, split s).
//
// What is computed: for the G = Hq/Hkv query heads that share KV head kvh
// (page "TensorRT对Grouped Query Attention的支持进展", section "技术演进背景"),
// softmax(scale * q K^T) V over the tokens of split s, evaluated page by page with an
// online softmax so that no score vector reaches memory (page
// "TensorRT-LLM与TensorRT核心差异解析", section 4.2.1). K/V rows are found through the
// page table (same two pages: section "动态形状与KV Cache管理" and section 4.2.2). The
// split partial format (normalised output + natural-log LSE) is the NumSplits
// decomposition of page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践", section
// "核心参数调优：PackGQA与NumSplits的协同舞蹈".
//
// MI355X design (VALU only: the path is HBM-bound for G <= 8):
//   * One (page, kv head) block is P*D contiguous elements, so every 128-bit wave load
//     moves 1 KiB contiguous. A token row of D elements spans one 16-lane DPP row: a
//     wave holds 4 tokens per load, each lane E = D/16 elements of its row.
//   * q.k partials are summed across the DPP row with quad_perm + row mirrors; bf16
//     pairs go through v_dot2_f32_bf16. Each DPP row keeps its own online-softmax state
//     (m, l, acc) over the tokens it sees (log2 domain, scale*log2(e) folded into the
//     exponent, lazily raised maximum); the 4 rows x 4 waves are merged once at the
//     end through LDS.
//   * G <= 8 (decode_regs_kernel): all G heads of the group live in one wave, so a K/V
//     row is loaded ONCE into VGPRs and used by every head of the group (repeat_kv is
//     never materialised). Each wave streams its own pages with the next page in
//     flight; waves never synchronise until the final merge, and no LDS limits the
//     bytes in flight.
//   * G >= 16 (decode_lds_kernel): the heads span several waves, so each K/V tile is
//     staged once in LDS (global_load_lds_dwordx4, double-buffered) and read by all of
//     them.
#include "decode_common.h"

namespace gqa {

// Merge the 4 rows x 4 waves of states through LDS and write the output (NS == 1) or the
// split partial (normalised output + natural-log LSE).
template <typename T, int D, int G>
__device__ __forceinline__ void merge_and_store(const WaveState<T, D, DecodeShape<T, D, G>::HW>& st,
                                                char* smem, int w, int r, int qd, int b, int kvh,
                                                int split, int Hq, int num_splits,
                                                T* __restrict__ out, float* __restrict__ ws_o,
                                                float* __restrict__ ws_lse) {
  using S = DecodeShape<T, D, G>;
  constexpr int HW = S::HW;
  float* acc_lds = (float*)smem;
  float* m_lds = acc_lds + S::NSTATE * D;
  float* l_lds = m_lds + S::NSTATE;
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const int si = (w * 4 + r) * HW + hw;
#pragma unroll
    for (int e = 0; e < S::E; ++e) acc_lds[si * D + lane_dim<T, D>(qd, e)] = st.acc[hw][e];
    if (qd == 0) {
      m_lds[si] = st.m[hw];
      l_lds[si] = st.l[hw];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += S::THREADS) {
    const int hl = idx / D;
    const int d = idx % D;
    const int hgi = hl / HW;
    const int hw = hl % HW;
    float M = -INFINITY;
    for (int t = 0; t < S::TG; ++t)
      for (int rr = 0; rr < 4; ++rr) M = fmaxf(M, m_lds[((hgi + S::HG * t) * 4 + rr) * HW + hw]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int t = 0; t < S::TG; ++t)
        for (int rr = 0; rr < 4; ++rr) {
          const int si = ((hgi + S::HG * t) * 4 + rr) * HW + hw;
          const float wgt = __builtin_amdgcn_exp2f(m_lds[si] - M);
          L += wgt * l_lds[si];
          A += wgt * acc_lds[si * D + d];
        }
    }
    const float o = (L > 0.f) ? A / L : 0.f;
    const int h = kvh * G + hl;
    if (ws_o == nullptr) {
      T* dst = out + ((size_t)b * Hq + h) * D + d;
      if constexpr (sizeof(T) == 2) {
        ((uint16_t*)dst)[0] = f32_to_bf16(o);
      } else {
        *dst = o;
      }
    } else {
      const size_t row = ((size_t)b * Hq + h) * num_splits + split;
      ws_o[row * D + d] = o;
      if (d == 0) ws_lse[row] = (L > 0.f) ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------------------
// G <= 8: one workgroup of 8 waves per (sequence, split, group of up to 8 KV heads).
// Wave w owns KV head w % KVW of the group (KVW = kv heads per workgroup, a power of
// two <= 8) and the split's pages w / KVW, w / KVW + 8 / KVW, ... It streams them
// straight into VGPRs with the next page in flight: no LDS staging, no barriers until
// the final merge. The waves of a group read the KVW neighbouring (page, kv head)
// blocks of the same physical page at about the same time, so DRAM sees KVW * 4 KiB
// contiguous per page instead of scattered 4 KiB blocks.
// ------------------------------------------------------------------------------------
constexpr int kRegsWaves = 8;
constexpr int kRegsThreads = kRegsWaves * kWave;

// NT: K/V rows read with the streaming hint (see launch_decode for when).
template <typename T, int D, int G, bool NT>
__global__ __launch_bounds__(kRegsThreads) void decode_regs_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv,
    int max_pages, int num_splits, int kvw, float scale_log2) {
  using S = DecodeShape<T, D, G>;
  static_assert(S::HG == 1, "all heads of the group in one wave");
  constexpr int HW = S::HW;
  constexpr int W32 = S::W32;
  constexpr int E = S::E;
  constexpr int SLOT = HW * D + 2 * HW;  // per wave: acc[HW][D], m[HW], l[HW]
  __shared__ float red[kRegsWaves * SLOT];

  const int groups = (Hkv + kvw - 1) / kvw;
  const int split = blockIdx.x / groups;
  const int grp = blockIdx.x % groups;
  const int b = blockIdx.y;
  const int w = wave_id();
  const int lane = lane_id();
  const int r = lane >> 4;
  const int qd = lane & 15;
  const int tgw = kRegsWaves / kvw;  // waves sharing one KV head (token groups)
  const int kvh = grp * kvw + w % kvw;
  const int tg = w / kvw;
  const bool active = kvh < Hkv;
  const SplitRange sr = split_range(context_lens, b, split, num_splits, max_pages);
  const int32_t* pt_row = page_table + (size_t)b * max_pages;
  const size_t page_stride = (size_t)Hkv * S::PAGE;
  const char* k_base = (const char*)k_cache + (size_t)kvh * S::PAGE + r * S::ROW;
  const char* v_base = (const char*)v_cache + (size_t)kvh * S::PAGE + r * S::ROW;

  WaveState<T, D, HW> st;
  st.init(q + ((size_t)b * Hq + (active ? kvh : 0) * G) * D, qd, scale_log2 < 0.f);

  uint32_t kb[2][4][W32], vb[2][4][W32];
  auto load_page = [&](int buf, int lp) {
    const size_t off = (size_t)pt_row[lp] * page_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (NT) {
        load_row_nt<T, D>(k_base + off + i * 4 * S::ROW, qd, kb[buf][i]);
        load_row_nt<T, D>(v_base + off + i * 4 * S::ROW, qd, vb[buf][i]);
      } else {
        load_row<T, D>(k_base + off + i * 4 * S::ROW, qd, kb[buf][i]);
        load_row<T, D>(v_base + off + i * 4 * S::ROW, qd, vb[buf][i]);
      }
    }
  };
  auto run = [&](int buf, int lp) {
    const int tok0 = lp * kPage + r;
    if (lp + 1 < sr.lp1) {
      st.template page<false>(kb[buf], vb[buf], tok0, sr.t_end, abs_scale(scale_log2));
    } else {
      st.template page<true>(kb[buf], vb[buf], tok0, sr.t_end, abs_scale(scale_log2));
    }
  };
  if (active) {
    // The prefetch is issued on every step (past the split it re-reads the current page,
    // an L2 hit) so the loads in flight are the same on every path and the wait before
    // each page is exactly "all but the newest page".
    int lp = sr.lp0 + tg;
    if (lp < sr.lp1) load_page(0, lp);
    for (; lp < sr.lp1; lp += 2 * tgw) {
      const int lp_b = lp + tgw;
      load_page(1, lp_b < sr.lp1 ? lp_b : lp);
      run(0, lp);
      if (lp_b >= sr.lp1) break;
      const int lp_c = lp_b + tgw;
      load_page(0, lp_c < sr.lp1 ? lp_c : lp_b);
      run(1, lp_b);
    }
  }

  // ---- merge the 4 DPP rows of each wave, then the token groups of each KV head
  // through LDS ----
  st.merge_rows();
  {
    float* slot = red + w * SLOT;
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      if (r == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) slot[hw * D + lane_dim<T, D>(qd, e)] = st.acc[hw][e];
      }
      if (lane == 0) {
        slot[HW * D + hw] = st.m[hw];
        slot[HW * D + HW + hw] = st.l[hw];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kvw * G * D; idx += kRegsThreads) {
    const int kl = idx / (G * D);
    const int hl = (idx / D) % G;
    const int d = idx % D;
    const int kv = grp * kvw + kl;
    if (kv >= Hkv) continue;
    float M = -INFINITY;
    for (int t = 0; t < tgw; ++t) M = fmaxf(M, red[(kl + kvw * t) * SLOT + HW * D + hl]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int t = 0; t < tgw; ++t) {
        const float* slot = red + (kl + kvw * t) * SLOT;
        const float wgt = __builtin_amdgcn_exp2f(slot[HW * D + hl] - M);
        L += wgt * slot[HW * D + HW + hl];
        A += wgt * slot[hl * D + d];
      }
    }
    const float o = (L > 0.f) ? A / L : 0.f;
    const int h = kv * G + hl;
    if (ws_o == nullptr) {
      T* dst = out + ((size_t)b * Hq + h) * D + d;
      if constexpr (sizeof(T) == 2) {
        ((uint16_t*)dst)[0] = f32_to_bf16(o);
      } else {
        *dst = o;
      }
    } else {
      const size_t row = ((size_t)b * Hq + h) * num_splits + split;
      ws_o[row * D + d] = o;
      if (d == 0) ws_lse[row] = (L > 0.f) ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------------------
// Any G (used for G >= 16): K/V tiles staged once in LDS and shared by all waves.
// ------------------------------------------------------------------------------------

// s_waitcnt vmcnt(n * LOADS) for a runtime n in [0, NST-2] (tail of the pipeline).
template <int LOADS, int NST>
__device__ __forceinline__ void wait_tiles(int n) {
  if (NST > 3 && n >= 2) {
    wait_vmcnt<(NST > 3 ? 2 * LOADS : 0)>();
  } else if (NST > 2 && n >= 1) {
    wait_vmcnt<(NST > 2 ? LOADS : 0)>();
  } else {
    wait_vmcnt<0>();
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_lds_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv,
    int max_pages, int num_splits, float scale_log2) {
  using S = DecodeShape<T, D, G>;
  constexpr int NP = S::NP;
  constexpr int W32 = S::W32;
  __shared__ __attribute__((aligned(16))) char smem[S::LDS_STAGED];

  const int split = blockIdx.x % num_splits;
  const int kvh = blockIdx.x / num_splits;
  const int b = blockIdx.y;
  const int w = wave_id();
  const int lane = lane_id();
  const int r = lane >> 4;
  const int qd = lane & 15;
  const int hg = w % S::HG;
  const int tg = w / S::HG;
  const SplitRange sr = split_range(context_lens, b, split, num_splits, max_pages);
  const int ntiles = (sr.lp1 - sr.lp0 + NP - 1) / NP;
  const int32_t* pt_row = page_table + (size_t)b * max_pages;
  const size_t page_stride = (size_t)Hkv * S::PAGE;
  const char* k_base = (const char*)k_cache + (size_t)kvh * S::PAGE;
  const char* v_base = (const char*)v_cache + (size_t)kvh * S::PAGE;

  WaveState<T, D, S::HW> st;
  st.init(q + ((size_t)b * Hq + kvh * G + hg * S::HW) * D, qd, scale_log2 < 0.f);

  // Page ids: scalar loads of the NEXT tile's ids go out with this tile's DMA, so the
  // issue path never waits on the page table. Entries past the split are replaced by
  // its last live page (re-read, then masked).
  int pid_next[NP];
  auto fetch_pids = [&](int tile) {
#pragma unroll
    for (int j = 0; j < NP; ++j) pid_next[j] = pt_row[min(sr.lp0 + tile * NP + j, sr.lp1 - 1)];
  };
  auto issue_tile = [&](int tile, int stg) {
    int pid[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) pid[j] = pid_next[j];
    if (tile + 1 < ntiles) fetch_pids(tile + 1);
    char* stage = smem + stg * S::STAGE;
#pragma unroll
    for (int k = 0; k < S::LOADS; ++k) {
      const int wave_chunk = k * S::THREADS + w * kWave;  // first 16-byte chunk of this wave
      const int blk = wave_chunk * 16 / S::PAGE;          // K pages 0..NP-1, V pages NP..2NP-1
      const int off = (wave_chunk * 16) % S::PAGE + lane * 16;
      const char* src = (blk < NP ? k_base : v_base) + (size_t)pid[blk % NP] * page_stride + off;
      lds_dma16(src, stage + wave_chunk * 16);
    }
  };
  auto compute_tile = [&](int tile, int stg, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* stage = smem + stg * S::STAGE;
#pragma unroll
    for (int j0 = 0; j0 < NP; j0 += S::TG) {
      const int j = j0 + tg;
      const int lp = sr.lp0 + tile * NP + j;
      if (j < NP && lp < sr.lp1) {
        uint32_t kw[4][W32], vw[4][W32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          load_row<T, D>(stage + j * S::PAGE + (4 * i + r) * S::ROW, qd, kw[i]);
          load_row<T, D>(stage + (NP + j) * S::PAGE + (4 * i + r) * S::ROW, qd, vw[i]);
        }
        st.template page<MASKED>(kw, vw, lp * kPage + r, sr.t_end, abs_scale(scale_log2));
      }
    }
  };

  // Stage handshake: wait for this wave's DMA of the tile, then a bare s_barrier (every
  // wave's DMA has landed). A full __syncthreads() would also drain the prefetch of the
  // following tiles, which must stay in flight during compute.
  if (ntiles > 0) fetch_pids(0);
  for (int t = 0; t < S::NST - 1; ++t)
    if (t < ntiles) issue_tile(t, t);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int stg = tile % S::NST;
    const int ahead = tile + S::NST - 1;
    if (ahead < ntiles) {
      issue_tile(ahead, ahead % S::NST);
      wait_vmcnt<(S::NST - 1) * S::LOADS>();
    } else {
      wait_tiles<S::LOADS, S::NST>(ntiles - 1 - tile);
    }
    __builtin_amdgcn_s_barrier();
    if (tile + 1 < ntiles) {
      compute_tile(tile, stg, std::false_type{});
    } else {
      compute_tile(tile, stg, std::true_type{});
    }
    // all reads of this stage done before a later DMA overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
  }
  __syncthreads();
  merge_and_store<T, D, G>(st, smem, w, r, qd, b, kvh, split, Hq, num_splits, out, ws_o, ws_lse);
}

// ------------------------------------------------------------------------------------
// bf16, G >= 16: the group's heads as the columns of matrix-core products. With 16 or 32
// query heads per KV head a page is a dense contraction (16 tokens x D dims x G heads), the
// packing of grouped heads into one matrix dimension that page "解锁GQA性能潜力：从批量大小
// 敏感性到高效优化实践" (section "核心参数调优：PackGQA与NumSplits的协同舞蹈") describes; on the
// vector ALU the 32-head case is bound by its dot products, not by HBM.
//
// K/V tiles (NP pages of K, then NP pages of V) stream into LDS by global_load_lds_dwordx4
// through an NST-stage ring (the DMA of the next NST - 1 tiles stays in flight during
// compute). Wave w takes pages w, w + 4, ... of a tile and, per page and per 16 heads:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16, D / 32 steps; A = K rows (ds_read_b128,
//                  16-byte chunks XOR-swizzled by row), B = q held in registers;
//                  lane l = 16 g + n gets tokens 4 g .. 4 g + 3 of head n;
//   softmax        lane-local per head n (log2 domain, lazily raised reference max);
//   O^T += V^T P^T v_mfma_f32_16x16x16_bf16, D / 16 dim tiles; A = V^T read transposed
//                  from the token-major tile (ds_read_b64_tr_b16), B = the lane's own
//                  weights as bf16 (the score layout is the B layout), so the output rows
//                  of a head stay in the lanes that own its softmax state.
// The 4 waves' states are merged through LDS at the end (output, or the split partial).
// ------------------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a raw buffer into LDS (buffer_load_dwordx4 ... lds, with the
// streaming hint: every K/V row is read once; lane i writes LDS bytes m0 + 16 i .. + 15).
// Issued from assembly so that the compiler does not track the
// LDS write: it would otherwise wait for every load in flight before each transpose read of
// LDS. The kernel orders the write itself (s_waitcnt vmcnt on the issuing wave, then a
// workgroup barrier) before any wave reads that stage.
__device__ __forceinline__ void dma16_untracked(u32x4_t rsrc, uint32_t voffset, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(m0)
               : "memory");
}
// Raw buffer descriptor over `bytes` bytes at a wave-uniform base.
__device__ __forceinline__ u32x4_t raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF),
                 bytes, 0x00020000u};
}

template <int D>
struct MqShape {
  static constexpr int ROW = D * 2;            // bytes per token row
  static constexpr int PAGE = kPage * ROW;     // bytes per (page, kv head) block
  static constexpr int CH = ROW / 16;          // 16-byte chunks per row
  static constexpr int NP = 4;                 // pages per tile (one per wave)
  static constexpr int STAGE = 2 * NP * PAGE;  // K pages, then V pages
  static constexpr int NST = D == 128 ? 4 : 6; // ring depth (128 / 96 KiB)
  static constexpr int LOADS = STAGE / (16 * kDecodeThreads);
  static constexpr int NC = D / 32;            // 32-dim steps of the score chain
  static constexpr int DT = D / 16;            // 16-dim tiles of the output
  static_assert(STAGE % (16 * kDecodeThreads) == 0 && (NST - 1) * LOADS < 64, "ring");
  // chunk swizzles: K rows are read 16 rows at one chunk, V rows 4 rows x 32 bytes
  static __device__ __forceinline__ int k_swz(int r) { return r & (CH - 1); }
  static __device__ __forceinline__ int v_swz(int r) { return ((r & (CH / 2 - 1)) << 1); }
};

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_mq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ context_lens, bf16_t* __restrict__ out,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv, int max_pages,
    int num_splits, float scale_log2) {
  using M = MqShape<D>;
  constexpr int NP = M::NP, NST = M::NST, NH = G / 16;
  static_assert(G % 16 == 0, "16 heads per product");
  constexpr int MERGE = kDecodeWaves * (G * (D + 4) + 2 * G) * 4;
  constexpr int LDS = NST * M::STAGE > MERGE ? NST * M::STAGE : MERGE;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  const uint32_t smem0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&smem[0];

  const int split = blockIdx.x % num_splits;
  const int kvh = blockIdx.x / num_splits;
  const int b = blockIdx.y;
  const int w = wave_id();
  const int lane = lane_id();
  const int n = lane & 15;   // head column (scores / PV B), token row (K reads)
  const int g = lane >> 4;   // token group: tokens 4g .. 4g + 3 of a page
  const SplitRange sr = split_range(context_lens, b, split, num_splits, max_pages);
  const int ntiles = (sr.lp1 - sr.lp0 + NP - 1) / NP;
  const int32_t* pt_row = page_table + (size_t)b * max_pages;
  const size_t page_stride = (size_t)Hkv * M::PAGE;
  const char* k_base = (const char*)k_cache + (size_t)kvh * M::PAGE;
  const char* v_base = (const char*)v_cache + (size_t)kvh * M::PAGE;
  const float sl2 = abs_scale(scale_log2);

  // q of head 16 h + n, dims 32 c + 8 g .. + 7 (the B operand of the score chain); a
  // negative scale is moved onto q (exact sign flips) and |scale| goes into the exponent.
  u32x4_t qb[NH][M::NC];
  {
    const uint32_t flip = scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const char* src = (const char*)(q + ((size_t)b * Hq + kvh * G + 16 * h + n) * D);
#pragma unroll
      for (int c = 0; c < M::NC; ++c) qb[h][c] = *(const u32x4_t*)(src + c * 64 + g * 16) ^ flip;
    }
  }
  float mrun[NH], lrun[NH];
  f32x4_t acc[NH][M::DT];  // O^T: dims 16 t + 4 g + j of head 16 h + n
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    mrun[h] = -INFINITY;
    lrun[h] = 0.f;
#pragma unroll
    for (int t = 0; t < M::DT; ++t) acc[h][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  int pid_next[NP];
  auto fetch_pids = [&](int tile) {
#pragma unroll
    for (int j = 0; j < NP; ++j) pid_next[j] = pt_row[min(sr.lp0 + tile * NP + j, sr.lp1 - 1)];
  };
  // DMA of one tile: lane i of a wave instruction fills 16 bytes at a fixed LDS position
  // (row r, chunk c of a page block) and fetches the chunk that belongs there, c ^ swz(r).
  auto issue_tile = [&](int tile, int stg) {
    int pid[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) pid[j] = pid_next[j];
    if (tile + 1 < ntiles) fetch_pids(tile + 1);
    const uint32_t stage = smem0 + stg * M::STAGE;
#pragma unroll
    for (int k = 0; k < M::LOADS; ++k) {
      const int wave_chunk = k * kDecodeThreads + w * kWave;
      const int blk = wave_chunk * 16 / M::PAGE;  // K pages 0..NP-1, V pages NP..2NP-1
      const int pos = (wave_chunk * 16) % M::PAGE + lane * 16;
      const int r = pos / M::ROW;
      const int c = (pos % M::ROW) / 16;
      const int src_c = c ^ (blk < NP ? M::k_swz(r) : M::v_swz(r));
      const u32x4_t rs = raw_rsrc((blk < NP ? k_base : v_base) +
                                      (size_t)pid[blk % NP] * page_stride, M::PAGE);
      dma16_untracked(rs, (uint32_t)(r * M::ROW + src_c * 16),
                      __builtin_amdgcn_readfirstlane(stage + wave_chunk * 16));
    }
  };

  auto page = [&](const char* kpage, const char* vpage, int tok0, bool masked) {
    // scores S^T = K Q^T for both head halves
    f32x4_t s[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) s[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < M::NC; ++c) {
      const u32x4_t ka = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
          kpage + n * M::ROW + (((4 * c + g) ^ M::k_swz(n)) << 4));
#pragma unroll
      for (int h = 0; h < NH; ++h)
        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                       __builtin_bit_cast(bf16x8_t, qb[h][c]),
                                                       s[h], 0, 0, 0);
    }
    // V^T operands (transposed reads), issued before the softmax so their latency overlaps it
    s16x4_t va[M::DT];
    {
      const int r = 4 * g + (n >> 2);
      const char* vrow = vpage + r * M::ROW + 8 * (n & 1);
#pragma unroll
      for (int t = 0; t < M::DT; ++t) {
        const int ch = 2 * t + ((n & 3) >> 1);
        va[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(vrow + ((ch ^ M::v_swz(r)) << 4)));
      }
    }
    float x[NH][4], mx[NH];
    bool trig = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[h][j] = s[h][j] * sl2;
        if (masked && tok0 + 4 * g + j >= sr.t_end) x[h][j] = -INFINITY;
      }
      mx[h] = fmaxf(fmaxf(x[h][0], x[h][1]), fmaxf(x[h][2], x[h][3]));
      trig |= mx[h] > mrun[h] + kLazyLog2;
    }
    // The reference max of a head (one value for the 4 token groups) is raised only when a
    // score exceeds it by more than 2^kLazyLog2; acc and l are rescaled then.
    if (__any(trig)) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float Mx = rows4_max(mx[h]);
        const float m_new = fmaxf(mrun[h], Mx);
        const float m_ref = (m_new > mrun[h] + kLazyLog2) ? m_new : mrun[h];
        const float alpha = (m_ref == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun[h] - m_ref);
        lrun[h] *= alpha;
        mrun[h] = m_ref;
#pragma unroll
        for (int t = 0; t < M::DT; ++t) acc[h][t] *= alpha;
      }
    }
    if (masked) {  // dead slots (tokens >= t_end) may hold NaN: never multiply them
#pragma unroll
      for (int t = 0; t < M::DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 4 * g + i >= sr.t_end) va[t][i] = 0;
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float msub = mrun[h] == -INFINITY ? 0.f : mrun[h];
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[h][j] - msub);
      lrun[h] += (p[0] + p[1]) + (p[2] + p[3]);
      const u32x2_t pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      const s16x4_t pb = __builtin_bit_cast(s16x4_t, pk);
#pragma unroll
      for (int t = 0; t < M::DT; ++t)
        acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[t], pb, acc[h][t], 0, 0, 0);
    }
  };

  auto compute_tile = [&](int tile, int stg, bool masked_tile) {
    const char* stage = smem + stg * M::STAGE;
#pragma unroll
    for (int j = w; j < NP; j += kDecodeWaves) {
      const int lp = sr.lp0 + tile * NP + j;
      if (lp < sr.lp1)
        page(stage + j * M::PAGE, stage + (NP + j) * M::PAGE, lp * kPage,
             masked_tile && lp + 1 == sr.lp1);
    }
  };

  if (ntiles > 0) fetch_pids(0);
  for (int t = 0; t < NST - 1; ++t)
    if (t < ntiles) issue_tile(t, t);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int stg = tile % NST;
    const int ahead = tile + NST - 1;
    if (ahead < ntiles) {
      issue_tile(ahead, ahead % NST);
      wait_vmcnt<(NST - 1) * M::LOADS>();
    } else {
      const int left = ntiles - 1 - tile;  // tiles still in flight after this one
      if (NST > 5 && left >= 4) wait_vmcnt<(NST > 5 ? 4 * M::LOADS : 0)>();
      else if (NST > 4 && left >= 3) wait_vmcnt<(NST > 4 ? 3 * M::LOADS : 0)>();
      else if (NST > 3 && left >= 2) wait_vmcnt<(NST > 3 ? 2 * M::LOADS : 0)>();
      else if (NST > 2 && left >= 1) wait_vmcnt<(NST > 2 ? M::LOADS : 0)>();
      else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    compute_tile(tile, stg, tile + 1 == ntiles);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  }

  // ---- merge the 4 waves through LDS: per wave m[h], l[h] (head-uniform after the group
  // sum) and O^T of all heads; then one thread per (head, dim) ----
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float lt = lrun[h];
    lt = rows4_sum(lt);
    lrun[h] = lt;
  }
  __syncthreads();
  constexpr int DP = D + 4;  // padded row: the 16 heads of a store land in different banks
  float* acc_lds = (float*)smem;                      // [wave][head][DP]
  float* m_lds = acc_lds + kDecodeWaves * G * DP;     // [wave][head]
  float* l_lds = m_lds + kDecodeWaves * G;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int hl = 16 * h + n;
#pragma unroll
    for (int t = 0; t < M::DT; ++t)
      *(f32x4_t*)&acc_lds[(w * G + hl) * DP + 16 * t + 4 * g] = acc[h][t];
    if (g == 0) {
      m_lds[w * G + hl] = mrun[h];
      l_lds[w * G + hl] = lrun[h];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int hl = idx / D, d = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) Mx = fmaxf(Mx, m_lds[ww * G + hl]);
    float L = 0.f, A = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kDecodeWaves; ++ww) {
        const float wgt = __builtin_amdgcn_exp2f(m_lds[ww * G + hl] - Mx);
        L += wgt * l_lds[ww * G + hl];
        A += wgt * acc_lds[(ww * G + hl) * DP + d];
      }
    }
    const float o = (L > 0.f) ? A / L : 0.f;
    const int hq = kvh * G + hl;
    if (ws_o == nullptr) {
      ((uint16_t*)out)[((size_t)b * Hq + hq) * D + d] = f32_to_bf16(o);
    } else {
      const size_t row = ((size_t)b * Hq + hq) * num_splits + split;
      ws_o[row * D + d] = o;
      if (d == 0) ws_lse[row] = (L > 0.f) ? (Mx + __builtin_log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// ---- host-side dispatch over (dtype, D, G) ----------------------------------------------

template <typename T, int D, int G>
static int launch_decode(const void* q, const void* k, const void* v, const int32_t* pt,
                         const int32_t* lens, void* out, float* ws_o, float* ws_lse, int B,
                         int Hq, int Hkv, int max_pages, int ns, float scale,
                         hipStream_t stream) {
  float* wo = ns > 1 ? ws_o : nullptr;
  float* wl = ns > 1 ? ws_lse : nullptr;
  if constexpr (G <= 8) {
    // One KV head per workgroup: its 8 waves take the split's pages round-robin. (Grouping
    // several KV heads per workgroup so that neighbouring (page, kv head) blocks are read
    // together measured no faster, and leaves small batches with too few workgroups.)
    // The streaming hint on the K/V loads: faster for G >= 2 at every split count measured
    // (long contexts by 10%), and for G = 1 without splits, but much slower for G = 1 with
    // splits (B = 256, Hkv = 32, T = 1024, 8 splits: 1225 vs 760 us), where every wave streams
    // only a few pages of one head.
    const int kvw = 1;
    const int groups = Hkv;
    if (G >= 2 || ns == 1) {
      hipLaunchKernelGGL((decode_regs_kernel<T, D, G, true>), dim3(groups * ns, B),
                         dim3(kRegsThreads), 0, stream, (const T*)q, (const T*)k, (const T*)v, pt,
                         lens, (T*)out, wo, wl, Hq, Hkv, max_pages, ns, kvw, scale * kLog2e);
    } else {
      hipLaunchKernelGGL((decode_regs_kernel<T, D, G, false>), dim3(groups * ns, B),
                         dim3(kRegsThreads), 0, stream, (const T*)q, (const T*)k, (const T*)v, pt,
                         lens, (T*)out, wo, wl, Hq, Hkv, max_pages, ns, kvw, scale * kLog2e);
    }
  } else if constexpr (sizeof(T) == 2) {
    // bf16, G >= 16: heads as matrix-core columns
    hipLaunchKernelGGL((decode_mq_kernel<D, G>), dim3(Hkv * ns, B), dim3(kDecodeThreads), 0,
                       stream, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, pt, lens,
                       (bf16_t*)out, wo, wl, Hq, Hkv, max_pages, ns, scale * kLog2e);
  } else {
    hipLaunchKernelGGL((decode_lds_kernel<T, D, G>), dim3(Hkv * ns, B), dim3(kDecodeThreads), 0,
                       stream, (const T*)q, (const T*)k, (const T*)v, pt, lens, (T*)out, wo, wl,
                       Hq, Hkv, max_pages, ns, scale * kLog2e);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <typename T, int D>
static int dispatch_group(int G, const void* q, const void* k, const void* v,
                          const int32_t* pt, const int32_t* lens, void* out, float* ws_o,
                          float* ws_lse, int B, int Hq, int Hkv, int max_pages, int ns,
                          float scale, hipStream_t s) {
  switch (G) {
    case 1: return launch_decode<T, D, 1>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    case 2: return launch_decode<T, D, 2>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    case 4: return launch_decode<T, D, 4>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    case 8: return launch_decode<T, D, 8>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    case 16: return launch_decode<T, D, 16>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    case 32: return launch_decode<T, D, 32>(q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_decode_paged(const void* q, const void* k, const void* v, const int32_t* pt,
                        const int32_t* lens, void* out, float* ws_o, float* ws_lse, int B,
                        int Hq, int Hkv, int D, int max_pages, int ns, float scale, int dtype,
                        hipStream_t s) {
  const int G = Hq / Hkv;
  if (dtype == GQA_BF16) {
    if (D == 128) return dispatch_group<bf16_t, 128>(G, q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    if (D == 64) return dispatch_group<bf16_t, 64>(G, q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
  } else {
    if (D == 128) return dispatch_group<float, 128>(G, q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
    if (D == 64) return dispatch_group<float, 64>(G, q, k, v, pt, lens, out, ws_o, ws_lse, B, Hq, Hkv, max_pages, ns, scale, s);
  }
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
