// Shared pieces of the paged GQA decode kernels (gfx950, wave64): tile geometry, the
// lane <-> dimension map, row loads and the per-wave online-softmax state.
//
// Layout facts used throughout: one (page, kv head) block of the pool is P*D contiguous
// elements; a token row of D elements spans one 16-lane DPP row, so a wave holds 4 token
// rows per 128-bit load and each lane E = D/16 elements of its row.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "../../include/gqa.h"

namespace gqa {

constexpr float kLazyLog2 = 8.0f;  // log2 headroom before the running max is raised
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr int kPage = 16;          // tokens per page

// LDS pipeline of decode_lds_kernel: bytes of K+V staged per tile and number of stages.
#ifndef GQA_DECODE_TILE_KIB
#define GQA_DECODE_TILE_KIB 32
#endif
#ifndef GQA_DECODE_STAGES
#define GQA_DECODE_STAGES 2
#endif

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int P = kPage;
  static constexpr int WAVES = kDecodeWaves;
  static constexpr int THREADS = kDecodeThreads;
  static constexpr int EB = (int)sizeof(T);
  static constexpr int E = D / 16;             // elements per lane per token row
  static constexpr int LB = E * EB;            // bytes per lane per token row: 8, 16 or 32
  static constexpr int W32 = LB / 4;           // 32-bit words per lane per token row
  static constexpr int ROW = D * EB;           // bytes per token row
  static constexpr int PAGE = P * ROW;         // bytes per (page, kv head) block
  static constexpr int HW = G < 8 ? G : 8;     // query heads per wave
  static constexpr int HG = G / HW;            // head groups across waves
  static constexpr int TG = WAVES / HG;        // token groups across waves
  static constexpr int NSTATE = WAVES * 4 * HW;  // (wave, row, head) softmax states
  static constexpr int MERGE = NSTATE * D * 4 + 2 * NSTATE * 4;
  // LDS-staged variant
  static constexpr int NP = (GQA_DECODE_TILE_KIB * 1024 / (2 * PAGE)) > 0
                                ? GQA_DECODE_TILE_KIB * 1024 / (2 * PAGE) : 1;  // pages per tile
  static constexpr int STAGE = 2 * NP * PAGE;  // K pages then V pages
  static constexpr int NST = GQA_DECODE_STAGES;
  static constexpr int LOADS = STAGE / (16 * THREADS);  // 16-byte DMA loads per thread per tile
  static constexpr int LDS_STAGED = (NST * STAGE > MERGE) ? NST * STAGE : MERGE;
  static_assert(NP >= 1 && STAGE % (16 * THREADS) == 0, "tile geometry");
  static_assert(NST >= 2 && NST <= 4 && (NST - 1) * LOADS < 64, "pipeline depth");
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

// One lane's E elements of a token row (LDS or global) as raw 32-bit words.
template <typename T, int D>
__device__ __forceinline__ void load_row(const char* row, int qd, uint32_t (&w)[D / 16 * sizeof(T) / 4]) {
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

// load_row from global memory with a streaming (non-temporal) hint on 16-byte lane loads:
// cache rows are read once, and the hint was measured to raise the decode's streaming rate
// by 11% on 16-bit caches (8-byte lane loads were slower with it, so they go without).
template <typename T, int D>
__device__ __forceinline__ void load_row_nt(const char* row, int qd,
                                            uint32_t (&w)[D / 16 * sizeof(T) / 4]) {
  constexpr int LB = D / 16 * (int)sizeof(T);
  if constexpr (LB == 8) {
    u32x2_t v = *(const u32x2_t*)(row + qd * 8);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (LB == 16) {
    u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(row + qd * 16));
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    u32x4_t a = __builtin_nontemporal_load((const u32x4_t*)(row + qd * 16));
    u32x4_t b = __builtin_nontemporal_load((const u32x4_t*)(row + D * 2 + qd * 16));
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  }
}

// Inverse of load_row: write one lane's E elements of a token row.
template <typename T, int D>
__device__ __forceinline__ void store_kv_row(char* row, int qd, const uint32_t (&w)[D / 16 * sizeof(T) / 4]) {
  constexpr int LB = D / 16 * (int)sizeof(T);
  if constexpr (LB == 8) {
    *(u32x2_t*)(row + qd * 8) = u32x2_t{w[0], w[1]};
  } else if constexpr (LB == 16) {
    *(u32x4_t*)(row + qd * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  } else {
    *(u32x4_t*)(row + qd * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
    *(u32x4_t*)(row + D * 2 + qd * 16) = u32x4_t{w[4], w[5], w[6], w[7]};
  }
}

// Online-softmax state of one wave: HW query heads x (this lane's E dims), one state per
// DPP row (the row's 16 lanes hold identical m and l). T: q / output element type; TKV:
// cache element type (T itself, or an 8-bit float with bf16 q).
template <typename T, int D, int HW, typename TKV = T>
struct WaveState {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr bool kFp8 = is_fp8<TKV>();
  static_assert(!kFp8 || kBf16, "8-bit caches are read with bf16 queries");
  static constexpr int E = D / 16;
  static constexpr int W32 = E * (int)sizeof(T) / 4;
  static constexpr int WKV = E * (int)sizeof(TKV) / 4;  // cache words per lane per row
  static constexpr int KROWS = 4, KWORDS = WKV;          // K words per lane per page
  uint32_t qw[HW][W32];
  float m[HW], l[HW], acc[HW][E];

  // neg: the caller's scale is negative; q is negated here (exact) and the kernel runs with
  // |scale| (see abs_scale), so the row max taken on raw q.k stays the max of the scaled
  // scores.
  __device__ __forceinline__ void init(const T* q_head0, int qd, bool neg) {
    const uint32_t flip = neg ? (kBf16 ? 0x80008000u : 0x80000000u) : 0u;
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      load_row<T, D>((const char*)(q_head0 + (size_t)hw * D), qd, qw[hw]);
#pragma unroll
      for (int x = 0; x < W32; ++x) qw[hw][x] ^= flip;
      m[hw] = -INFINITY;
      l[hw] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hw][e] = 0.f;
    }
  }

  // Merge the 4 DPP rows into one state per head: afterwards every lane holds the merged
  // m, l and the merged acc of its row-column's dims. The whole wave must be active.
  __device__ __forceinline__ void merge_rows() {
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      const float M = rows4_max(m[hw]);
      const float wgt = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[hw] - M);
      const float lw = rows4_sum(l[hw] * wgt);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hw][e] = rows4_sum(acc[hw][e] * wgt);
      m[hw] = M;
      l[hw] = lw;
    }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      m[hw] = -INFINITY;
      l[hw] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hw][e] = 0.f;
    }
  }

  // Consume one page: this lane holds rows kw[i], vw[i] of tokens tok0 + 4*i (i < 4).
  // MASKED: tokens >= t_end are dead (their slots may hold anything, NaN included).
  template <bool MASKED>
  __device__ __forceinline__ void page(const uint32_t (&kw)[4][WKV], uint32_t (&vw)[4][WKV],
                                       int tok0, int t_end, float scale_log2) {
    float s[4][HW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t kb16[kFp8 ? W32 : 1];  // an 8-bit K row widened to bf16 pairs (exact)
      if constexpr (kFp8) {
#pragma unroll
        for (int x = 0; x < WKV; ++x) {
          kb16[2 * x] = fp8x2_to_bf16x2<TKV>(kw[i][x], false);
          kb16[2 * x + 1] = fp8x2_to_bf16x2<TKV>(kw[i][x], true);
        }
      }
#pragma unroll
      for (int hw = 0; hw < HW; ++hw) {
        float part = 0.f;
        if constexpr (kFp8) {
#pragma unroll
          for (int x = 0; x < W32; ++x) part = dot2_bf16(qw[hw][x], kb16[x], part);
        } else if constexpr (kBf16) {
#pragma unroll
          for (int x = 0; x < W32; ++x) part = dot2_bf16(qw[hw][x], kw[i][x], part);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e)
            part = fmaf(__uint_as_float(qw[hw][e]), __uint_as_float(kw[i][e]), part);
        }
        s[i][hw] = row16_sum(part);  // raw q.k; scale * log2(e) is applied in the exponent
      }
    }
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      valid[i] = !MASKED || (tok0 + 4 * i < t_end);
      if (!valid[i]) {
#pragma unroll
        for (int hw = 0; hw < HW; ++hw) s[i][hw] = -INFINITY;
#pragma unroll
        for (int x = 0; x < WKV; ++x) vw[i][x] = 0u;  // never multiply a dead slot
      }
    }
    // The reference max m is raised lazily, only when a new score exceeds it by more
    // than 2^kLazyLog2: acc is rarely rescaled, p <= 2^kLazyLog2 stays well inside
    // fp32, and acc / l is unchanged.
    float p[4][HW];
    float alpha[HW];
    bool rescale = false;
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      const float mx = fmaxf(fmaxf(s[0][hw], s[1][hw]), fmaxf(s[2][hw], s[3][hw])) * scale_log2;
      const float m_new = fmaxf(m[hw], mx);
      const float m_ref = (m_new > m[hw] + kLazyLog2) ? m_new : m[hw];
      const float m_sub = (MASKED && m_ref == -INFINITY) ? 0.f : m_ref;
      alpha[hw] = __builtin_amdgcn_exp2f(m[hw] - m_sub);
      rescale |= alpha[hw] != 1.0f;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i][hw] = __builtin_amdgcn_exp2f(fmaf(s[i][hw], scale_log2, -m_sub));
        psum += p[i][hw];
      }
      l[hw] = l[hw] * alpha[hw] + psum;
      m[hw] = m_ref;
    }
    if (__any(rescale)) {
#pragma unroll
      for (int hw = 0; hw < HW; ++hw)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hw][e] *= alpha[hw];
    }
    if constexpr (kBf16) {
      // PV on bf16 pairs: this lane holds rows i = 0..3 (tokens tok0 + 4i) of the page, so
      // for tokens (2j, 2j+1) and each of its dims the two V values are repacked into one
      // bf16 pair (v_perm_b32) and v_dot2_f32_bf16 adds p_2j v_2j + p_2j+1 v_2j+1 with P
      // rounded to bf16 (fp32 accumulation; l keeps the unrounded p).
      uint32_t vb16[4][W32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (kFp8) {
#pragma unroll
          for (int x = 0; x < WKV; ++x) {
            vb16[i][2 * x] = fp8x2_to_bf16x2<TKV>(vw[i][x], false);
            vb16[i][2 * x + 1] = fp8x2_to_bf16x2<TKV>(vw[i][x], true);
          }
        } else {
#pragma unroll
          for (int x = 0; x < W32; ++x) vb16[i][x] = vw[i][x];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t pp[HW];
#pragma unroll
        for (int hw = 0; hw < HW; ++hw) pp[hw] = pack_bf16x2(p[2 * j][hw], p[2 * j + 1][hw]);
#pragma unroll
        for (int x = 0; x < W32; ++x) {
          // (dim 2x of token 2j, of token 2j+1) and (dim 2x+1 of each)
          const uint32_t lo = __builtin_amdgcn_perm(vb16[2 * j + 1][x], vb16[2 * j][x], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(vb16[2 * j + 1][x], vb16[2 * j][x], 0x07060302u);
#pragma unroll
          for (int hw = 0; hw < HW; ++hw) {
            acc[hw][2 * x] = dot2_bf16(pp[hw], lo, acc[hw][2 * x]);
            acc[hw][2 * x + 1] = dot2_bf16(pp[hw], hi, acc[hw][2 * x + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float vf[E];
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = __uint_as_float(vw[i][e]);
#pragma unroll
        for (int hw = 0; hw < HW; ++hw)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[hw][e] = fmaf(p[i][hw], vf[e], acc[hw][e]);
      }
    }
  }
};

// The scale the kernels run with: |scale * log2 e| (a negative scale is moved onto q by
// WaveState::init), raised to 1e-30 so that dead slots (-inf) still give exp2 = 0 when the
// caller's scale is 0 (every live weight is then exp2(~0) = 1, the uniform weights of 0).
__device__ __forceinline__ float abs_scale(float scale_log2) {
  return fmaxf(fabsf(scale_log2), 1e-30f);
}

// Page-aligned token range of split `split` of sequence b: pages [lp0, lp1), tokens < t_end.
struct SplitRange {
  int lp0, lp1, t_end;
};
__device__ __forceinline__ SplitRange split_range(const int32_t* __restrict__ context_lens,
                                                  int b, int split, int num_splits,
                                                  int max_pages) {
  int T_b = context_lens[b];
  T_b = T_b < 0 ? 0 : (T_b > max_pages * kPage ? max_pages * kPage : T_b);
  const int n_pages = (T_b + kPage - 1) / kPage;
  const int per_split = (n_pages + num_splits - 1) / num_splits;
  SplitRange sr;
  sr.lp0 = min(split * per_split, n_pages);
  sr.lp1 = min(sr.lp0 + per_split, n_pages);
  sr.t_end = min(sr.lp1 * kPage, T_b);
  return sr;
}

}  // namespace gqa
