// Paged GQA decode on gfx950: one workgroup per (sequence b, KV head kvh, split s).
//
// What is computed: for the G = Hq/Hkv query heads that share KV head kvh
// (page "TensorRT对Grouped Query Attention的支持进展", section "技术演进背景"),
// softmax(scale * q K^T) V over the tokens of split s, evaluated tile by tile
// with an online softmax so that no score vector reaches memory (page
// "TensorRT-LLM与TensorRT核心差异解析", section 4.2.1). K/V rows are found through
// the page table (same two pages: section "动态形状与KV Cache管理" and section
// 4.2.2). The split partial format (normalised output + natural-log LSE) is the
// NumSplits decomposition of page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践",
// section "核心参数调优：PackGQA与NumSplits的协同舞蹈".
//
// MI355X design:
//   * K/V tiles (NP pages of K and NP pages of V, 32 KiB) move HBM -> LDS with
//     global_load_lds_dwordx4: 128-bit per lane, one (page, kv head) block is
//     P*D contiguous elements, so every wave instruction reads 1 KiB
//     contiguous. Two stages: the next tile streams in while this one is used.
//   * Each tile is staged ONCE and read from LDS by every query head of the
//     group: the repeat_kv expansion never exists anywhere.
//   * VALU only (the path is HBM-bound at G <= 8): a token row of D elements
//     spans one 16-lane DPP row, 4 tokens per wave instruction; q.k partials
//     are summed across the row with DPP (quad_perm + row mirrors), bf16 pairs
//     use v_dot2_f32_bf16. Each DPP row keeps its own online-softmax state
//     (m, l, acc) over the tokens it sees; the 4 rows x 4 waves are merged once
//     at the end through LDS.
//   * Scores are kept in the log2 domain (scale * log2 e folded in) so the
//     exponentials are v_exp_f32.
#include <type_traits>

#include "device_common.h"
#include "../../include/gqa.h"

namespace gqa {

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int P = 16;
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EB = (int)sizeof(T);
  static constexpr int E = D / 16;             // elements per lane per token row
  static constexpr int LB = E * EB;            // bytes per lane per token row: 8, 16 or 32
  static constexpr int ROW = D * EB;           // bytes per token row
  static constexpr int PAGE = P * ROW;         // bytes per (page, kv head) block
  static constexpr int NP = 16384 / PAGE;      // pages per tile (16 KiB of K, 16 KiB of V)
  static constexpr int STAGE = 2 * NP * PAGE;  // 32 KiB
  static constexpr int LOADS = STAGE / (16 * THREADS);  // 16-byte DMA loads per thread per tile
  static constexpr int HW = G < 8 ? G : 8;     // query heads per wave
  static constexpr int HG = G / HW;            // head groups across waves
  static constexpr int TG = WAVES / HG;        // token groups across waves
  static constexpr int NSTATE = WAVES * 4 * HW;  // (wave, row, head) softmax states
  static constexpr int MERGE = NSTATE * D * 4 + 2 * NSTATE * 4;
  static constexpr int LDS = (2 * STAGE > MERGE) ? 2 * STAGE : MERGE;
  static_assert(NP >= 1 && STAGE % (16 * THREADS) == 0, "tile geometry");
  static_assert(LB == 8 || LB == 16 || LB == 32, "lane geometry");
  static_assert(G % HW == 0 && WAVES % HG == 0, "head split");
};

// Dimension held in slot e of a lane with row-column qd (same map for q, K, V, out).
template <typename T, int D>
__device__ __forceinline__ int lane_dim(int qd, int e) {
  constexpr int E = D / 16;
  constexpr int LB = E * (int)sizeof(T);
  if constexpr (LB <= 16) {
    return qd * E + e;
  } else {
    return (e / 4) * (D / 2) + qd * 4 + (e % 4);
  }
}

// Load one lane's E elements of a token row from LDS as raw 32-bit words.
template <typename T, int D>
__device__ __forceinline__ void lds_row(const char* row, int qd, uint32_t (&w)[D / 16 * sizeof(T) / 4]) {
  constexpr int LB = D / 16 * (int)sizeof(T);
  if constexpr (LB == 8) {
    u32x2_t v = *(const u32x2_t*)(row + qd * 8);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (LB == 16) {
    u32x4_t v = *(const u32x4_t*)(row + qd * 16);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    u32x4_t a = *(const u32x4_t*)(row + qd * 16);
    u32x4_t b = *(const u32x4_t*)(row + D * 2 + qd * 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_paged_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ context_lens,
    T* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv,
    int max_pages, int num_splits, float scale_log2) {
  using S = DecodeShape<T, D, G>;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int E = S::E;
  constexpr int W32 = S::LB / 4;  // 32-bit words per lane per row
  constexpr int HW = S::HW;
  constexpr int P = S::P;
  constexpr int NP = S::NP;

  __shared__ __attribute__((aligned(16))) char smem[S::LDS];

  const int split = blockIdx.x % num_splits;
  const int kvh = blockIdx.x / num_splits;
  const int b = blockIdx.y;
  const int w = wave_id();
  const int lane = lane_id();
  const int r = lane >> 4;   // DPP row = token within a group of 4
  const int qd = lane & 15;  // column within the row
  const int hg = w % S::HG;
  const int tg = w / S::HG;

  int T_b = context_lens[b];
  T_b = T_b < 0 ? 0 : (T_b > max_pages * P ? max_pages * P : T_b);
  const int n_pages = (T_b + P - 1) / P;
  const int per_split = (n_pages + num_splits - 1) / num_splits;
  const int lp0 = min(split * per_split, n_pages);
  const int lp1 = min(lp0 + per_split, n_pages);
  const int t_end = min(lp1 * P, T_b);
  const int ntiles = (lp1 - lp0 + NP - 1) / NP;

  const int32_t* pt_row = page_table + (size_t)b * max_pages;
  const size_t page_stride = (size_t)Hkv * S::PAGE;
  const char* k_base = (const char*)k_cache + (size_t)kvh * S::PAGE;
  const char* v_base = (const char*)v_cache + (size_t)kvh * S::PAGE;

  // ---- q for this wave's heads, in this lane's dimension slots ----
  const int h_first = kvh * G + hg * HW;
  uint32_t qw[HW][W32];
  float qf[HW][E];
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const char* qrow = (const char*)(q + ((size_t)b * Hq + h_first + hw) * D);
    if constexpr (S::LB == 8) {
      u32x2_t v = *(const u32x2_t*)(qrow + qd * 8);
      qw[hw][0] = v[0]; qw[hw][1] = v[1];
    } else if constexpr (S::LB == 16) {
      u32x4_t v = *(const u32x4_t*)(qrow + qd * 16);
      for (int i = 0; i < 4; ++i) qw[hw][i] = v[i];
    } else {
      u32x4_t a = *(const u32x4_t*)(qrow + qd * 16);
      u32x4_t c = *(const u32x4_t*)(qrow + D * 2 + qd * 16);
      for (int i = 0; i < 4; ++i) { qw[hw][i] = a[i]; qw[hw][4 + i] = c[i]; }
    }
    if constexpr (!kBf16) {
      for (int e = 0; e < E; ++e) qf[hw][e] = __uint_as_float(qw[hw][e]) * scale_log2;
    }
  }

  float m[HW], l[HW], acc[HW][E];
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    m[hw] = -INFINITY;
    l[hw] = 0.f;
    for (int e = 0; e < E; ++e) acc[hw][e] = 0.f;
  }

  // ---- HBM -> LDS: tile t into stage st (wave-uniform page per instruction) ----
  auto issue_tile = [&](int tile, int st) {
    char* stage = smem + st * S::STAGE;
    const int base_lp = lp0 + tile * NP;
#pragma unroll
    for (int k = 0; k < S::LOADS; ++k) {
      const int wave_chunk = k * S::THREADS + w * kWave;  // first 16-byte chunk of this wave
      const int blk = wave_chunk * 16 / S::PAGE;          // K pages 0..NP-1, V pages NP..2NP-1
      const int off = (wave_chunk * 16) % S::PAGE + lane * 16;
      int lp = base_lp + (blk % NP);
      lp = lp < lp1 ? lp : lp1 - 1;  // past the split: re-read a live page, masked later
      const int phys = pt_row[lp];
      const char* src = (blk < NP ? k_base : v_base) + (size_t)phys * page_stride + off;
      lds_dma16(src, stage + wave_chunk * 16);
    }
  };

  // ---- one tile of this wave's pages ----
  auto compute_tile = [&](int tile, int st, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* stage = smem + st * S::STAGE;
    for (int j = tg; j < NP; j += S::TG) {
      const int lp = lp0 + tile * NP + j;
      if (lp >= lp1) break;
      const char* kp = stage + j * S::PAGE;
      const char* vp = stage + (NP + j) * S::PAGE;
      float s[4][HW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t kw[W32];
        lds_row<T, D>(kp + (4 * i + r) * S::ROW, qd, kw);
#pragma unroll
        for (int hw = 0; hw < HW; ++hw) {
          float part = 0.f;
          if constexpr (kBf16) {
#pragma unroll
            for (int x = 0; x < W32; ++x) part = dot2_bf16(qw[hw][x], kw[x], part);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) part = fmaf(qf[hw][e], __uint_as_float(kw[e]), part);
          }
          part = row16_sum(part);
          s[i][hw] = kBf16 ? part * scale_log2 : part;
        }
      }
      bool valid[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        valid[i] = !MASKED || (lp * P + 4 * i + r < t_end);
        if (!valid[i]) {
          for (int hw = 0; hw < HW; ++hw) s[i][hw] = -INFINITY;
        }
      }
      float p[4][HW];
#pragma unroll
      for (int hw = 0; hw < HW; ++hw) {
        const float mx = fmaxf(fmaxf(s[0][hw], s[1][hw]), fmaxf(s[2][hw], s[3][hw]));
        const float m_new = fmaxf(m[hw], mx);
        const float m_use = (MASKED && m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[hw] - m_use);
        float psum = 0.f;
        for (int i = 0; i < 4; ++i) {
          p[i][hw] = __builtin_amdgcn_exp2f(s[i][hw] - m_use);
          psum += p[i][hw];
        }
        l[hw] = l[hw] * alpha + psum;
        m[hw] = m_new;
        for (int e = 0; e < E; ++e) acc[hw][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t vw[W32];
        lds_row<T, D>(vp + (4 * i + r) * S::ROW, qd, vw);
        if (MASKED && !valid[i]) {
          for (int x = 0; x < W32; ++x) vw[x] = 0u;  // never multiply a dead slot (may be NaN)
        }
        float vf[E];
        if constexpr (kBf16) {
          for (int x = 0; x < W32; ++x) {
            vf[2 * x] = bf16lo_to_f32(vw[x]);
            vf[2 * x + 1] = bf16hi_to_f32(vw[x]);
          }
        } else {
          for (int e = 0; e < E; ++e) vf[e] = __uint_as_float(vw[e]);
        }
#pragma unroll
        for (int hw = 0; hw < HW; ++hw)
          for (int e = 0; e < E; ++e) acc[hw][e] = fmaf(p[i][hw], vf[e], acc[hw][e]);
      }
    }
  };

  // Stage handshake: wait for this wave's DMA of the tile, then a bare s_barrier
  // (every wave's DMA has landed). A full __syncthreads() would also drain the
  // prefetch of the next tile, which must stay in flight during compute.
  if (ntiles > 0) issue_tile(0, 0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int st = tile & 1;
    if (tile + 1 < ntiles) {
      issue_tile(tile + 1, st ^ 1);
      wait_vmcnt<S::LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (tile + 1 < ntiles) {
      compute_tile(tile, st, std::false_type{});
    } else {
      compute_tile(tile, st, std::true_type{});
    }
    // all reads of stage st done before the next iteration's DMA overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
  }
  __syncthreads();

  // ---- merge the (wave, row) states through LDS ----
  float* acc_lds = (float*)smem;
  float* m_lds = acc_lds + S::NSTATE * D;
  float* l_lds = m_lds + S::NSTATE;
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const int si = (w * 4 + r) * HW + hw;
    for (int e = 0; e < E; ++e) acc_lds[si * D + lane_dim<T, D>(qd, e)] = acc[hw][e];
    if (qd == 0) {
      m_lds[si] = m[hw];
      l_lds[si] = l[hw];
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
      if constexpr (kBf16) {
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

// ---- host-side dispatch over (dtype, D, G) ----------------------------------------------

template <typename T, int D, int G>
static int launch_decode(const void* q, const void* k, const void* v, const int32_t* pt,
                         const int32_t* lens, void* out, float* ws_o, float* ws_lse, int B,
                         int Hq, int Hkv, int max_pages, int ns, float scale,
                         hipStream_t stream) {
  dim3 grid(Hkv * ns, B);
  hipLaunchKernelGGL((decode_paged_kernel<T, D, G>), grid, dim3(256), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, pt, lens, (T*)out, ns > 1 ? ws_o : nullptr,
                     ns > 1 ? ws_lse : nullptr, Hq, Hkv, max_pages, ns, scale * kLog2e);
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
