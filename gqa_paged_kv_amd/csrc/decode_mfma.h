// Decode wave state with the scores on the matrix core (bf16 queries; bf16 or 8-bit cache).
//
// The G query heads that share a KV head are the columns of one small product, the packing
// of grouped heads into a matrix dimension that page "解锁GQA性能潜力：从批量大小敏感性到高效
// 优化实践" (section "核心参数调优：PackGQA与NumSplits的协同舞蹈") describes: per page,
// S^T = K_page Q^T is one chain of v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns,
// 32 dims per step), the columns holding the group's heads repeated 16 / min(G, 4) times
// (G = 8 takes two chains). That replaces the per-lane dot products and 16-lane DPP
// reductions of the vector path; what the wave still does on the VALU is the softmax of
// its own 4 scores per head and the PV products.
//
// Lane l (n = l % 16, g = l / 16):
//   * K operand: token row k_row(l) = (n / 4) + 4 (n % 4) of the page, dims q_dim(l, c) .. +8
//     of chunk c (the row permutation makes output row 4g + j the token g + 4j);
//   * Q operand: head p*GQ + n % GQ of pass p, the same dims;
//   * scores: tokens g + 4j (j < 4) of head p*GQ + n % GQ;
//   * PV: V rows g + 4i (i < 4), dims of lane_dim(n, e), all G heads: the weights of the
//     other heads come from the lanes of the same quad (DPP quad broadcast). 8-bit caches
//     (whose pages carry half the bytes for the same arithmetic, which the vector PV then
//     bounds): O^T += V^T P^T on the matrix core instead, one v_mfma_f32_16x16x16_bf16 per
//     16 dims of a page and score chain, K = the page's 16 tokens in the scores' order
//     4g + i <-> token g + 4i, so that B = P^T is the lane's own four weights and A = V^T
//     the lane's own rows (block e: dim lane_dim(n, e)); lane l then holds dims
//     lane_dim(4g + j, e) of its column's head, rearranged through LDS by merge_rows.
// The running max is one value per head for the whole wave (raised lazily, as in the
// vector path, by a wave-wide reduction only when some score exceeds it by 2^8), so the
// rows of the wave need no rescaling when they are merged.
#pragma once

#include "decode_common.h"

namespace gqa {

typedef short s16x4_mq __attribute__((ext_vector_type(4)));  // 4 bf16 operand bits

template <int H>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, H * 0x55, 0xF, 0xF, false);
}
// lane h of each quad to the whole quad (h must fold to a constant)
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x, int h) {
  switch (h) {
    case 0: return quad_bcast<0>(x);
    case 1: return quad_bcast<1>(x);
    case 2: return quad_bcast<2>(x);
    default: return quad_bcast<3>(x);
  }
}
__device__ __forceinline__ float quad_bcast(float x, int h) {
  return __uint_as_float(quad_bcast(__float_as_uint(x), h));
}

template <typename T, int D, int G, typename TKV = T>
struct WaveStateMq {
  static_assert(sizeof(T) == 2, "bf16 queries");
  static constexpr bool kFp8 = is_fp8<TKV>();
  static constexpr int GQ = G < 4 ? G : 4;  // heads per score chain (one per quad lane)
  static constexpr int NPASS = G / GQ;
  static constexpr int NC = D / 32;         // 32-dim steps of the score chain
  static constexpr int KROWS = NC;          // K words per lane per page: KROWS x KWORDS
  static constexpr int KWORDS = kFp8 ? 2 : 4;
  static constexpr int E = D / 16;          // PV dims per lane
  static constexpr int W32 = E / 2;         // bf16 words of a V row per lane
  static constexpr int WKV = kFp8 ? W32 / 2 : W32;
  static constexpr bool kPvMfma = kFp8;     // PV on the matrix core
  static constexpr int STAGE_FLOATS = kPvMfma ? G * D : 0;  // LDS per wave for merge_rows
  static_assert(D % 32 == 0 && G % GQ == 0 && NPASS <= 2, "shape");

  u32x4_t qb[NPASS][NC];
  float mrun[NPASS], lrun[NPASS];  // this lane's head: reference max, this row's sum
  f32x4_t accm[kPvMfma ? NPASS : 1][kPvMfma ? E : 1];  // matrix-core PV: O^T blocks
  float acc[G][E];                 // vector PV; matrix-core PV: valid after merge_rows()
  float m[G], l[G];                // per head, valid after merge_rows()

  static __device__ __forceinline__ int k_row(int lane) {
    const int n = lane & 15;
    return (n >> 2) + 4 * (n & 3);
  }
  // Dims of score step c taken by lane group g = lane / 16 (8 of them, contiguous): 16-bit
  // caches: c * 32 + g * 8; 8-bit caches: steps 2m and 2m + 1 share one 16-byte load of dims
  // m * 64 + g * 16 .. + 16, the first 8 for step 2m, the other 8 for step 2m + 1 (the score
  // is a sum over all dims, so Q only has to follow the same order).
  static __device__ __forceinline__ int q_dim(int lane, int c) {
    return kFp8 ? (c >> 1) * 64 + (lane >> 4) * 16 + (c & 1) * 8 : c * 32 + (lane >> 4) * 8;
  }
  // byte offset in a K row of 16-byte load c (8-bit: NC / 2 loads, 16-bit: NC)
  static __device__ __forceinline__ int k_off(int lane, int c) {
    return kFp8 ? c * 64 + (lane >> 4) * 16 : c * 64 + (lane >> 4) * 16;
  }
  static_assert(!kFp8 || NC % 2 == 0, "8-bit K rows are read 64 dims at a time");
  // this lane's words of K row `row` (the row k_row(lane) of a page), by 16-byte loads with
  // the streaming hint (see load_row_nt)
  static __device__ __forceinline__ void load_k(const char* row, int lane,
                                                uint32_t (&kw)[KROWS][KWORDS]) {
    if constexpr (kFp8) {
#pragma unroll
      for (int m = 0; m < NC / 2; ++m) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(row + k_off(lane, m)));
        kw[2 * m][0] = v[0]; kw[2 * m][1] = v[1];
        kw[2 * m + 1][0] = v[2]; kw[2 * m + 1][1] = v[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(row + k_off(lane, c)));
        kw[c][0] = v[0]; kw[c][1] = v[1]; kw[c][2] = v[2]; kw[c][3] = v[3];
      }
    }
  }
  static __device__ __forceinline__ void store_k(char* row, int lane,
                                                 const uint32_t (&kw)[KROWS][KWORDS]) {
    if constexpr (kFp8) {
#pragma unroll
      for (int m = 0; m < NC / 2; ++m)
        *(u32x4_t*)(row + k_off(lane, m)) =
            u32x4_t{kw[2 * m][0], kw[2 * m][1], kw[2 * m + 1][0], kw[2 * m + 1][1]};
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        *(u32x4_t*)(row + k_off(lane, c)) = u32x4_t{kw[c][0], kw[c][1], kw[c][2], kw[c][3]};
    }
  }

  // q_head0: the group's first query head. neg: the caller's scale is negative; q is
  // negated here (exact) and the kernel runs with |scale|.
  __device__ __forceinline__ void init(const T* q_head0, int lane, bool neg) {
    fetch_q(q_head0, lane, neg, qb);
    reset();
  }
  // This lane's Q operand words of a group into `dst` (qb itself, or a staging copy for a
  // unit that starts later).
  static __device__ __forceinline__ void fetch_q(const T* q_head0, int lane, bool neg,
                                                 u32x4_t (&dst)[NPASS][NC]) {
    const uint32_t flip = neg ? 0x80008000u : 0u;
    const int n = lane & 15;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const char* src = (const char*)(q_head0 + (size_t)(p * GQ + n % GQ) * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4_t v = *(const u32x4_t*)(src + q_dim(lane, c) * 2);
        dst[p][c] = v ^ flip;
      }
    }
  }
  // init() from Q words fetched earlier by fetch_q.
  __device__ __forceinline__ void init_from(const u32x4_t (&src)[NPASS][NC]) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
      for (int c = 0; c < NC; ++c) qb[p][c] = src[p][c];
    reset();
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      mrun[p] = -INFINITY;
      lrun[p] = 0.f;
    }
    if constexpr (kPvMfma) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p)
#pragma unroll
        for (int e = 0; e < E; ++e) accm[p][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }
  }

  // Merge the 4 rows (token groups) of the wave: every lane gets, for all G heads, the
  // group's m, l and the summed acc of its dims. The whole wave must be active.
  // stage: this wave's STAGE_FLOATS floats of LDS (matrix-core PV only): the lanes of the
  // first GQ columns write their head's O^T blocks as [head][e][16 rows], and every lane
  // reads back dims lane_dim(n, e) = n E + e of every head (row n of block e). One wave
  // writes and reads its own area, and LDS instructions of a wave complete in order.
  __device__ __forceinline__ void merge_rows(float* stage = nullptr) {
    float lt[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      lt[p] = rows4_sum(lrun[p]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = quad_bcast(mrun[h / GQ], h % GQ);
      l[h] = quad_bcast(lt[h / GQ], h % GQ);
    }
    if constexpr (kPvMfma) {
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const int n = lane & 15, g = lane >> 4;
      if (n < GQ) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
#pragma unroll
          for (int e = 0; e < E; ++e)
            *(f32x4_t*)(stage + ((p * GQ + n) * E + e) * 16 + 4 * g) = accm[p][e];
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = stage[(h * E + e) * 16 + n];
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = rows4_sum(acc[h][e]);
    }
  }

  // Consume one page. kw: this lane's K words (row k_row(lane)); vw[i]: V row g + 4i.
  // tok0 = page start + g. MASKED: tokens >= t_end are dead (their slots may hold anything).
  template <bool MASKED>
  __device__ __forceinline__ void page(const uint32_t (&kw)[KROWS][KWORDS],
                                       uint32_t (&vw)[4][WKV], int tok0, int t_end,
                                       float scale_log2) {
    f32x4_t s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) s[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4_t a;
      if constexpr (kFp8) {
        a = u32x4_t{fp8x2_to_bf16x2<TKV>(kw[c][0], false), fp8x2_to_bf16x2<TKV>(kw[c][0], true),
                    fp8x2_to_bf16x2<TKV>(kw[c][1], false), fp8x2_to_bf16x2<TKV>(kw[c][1], true)};
      } else {
        a = u32x4_t{kw[c][0], kw[c][1], kw[c][2], kw[c][3]};
      }
#pragma unroll
      for (int p = 0; p < NPASS; ++p)
        s[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, qb[p][c]),
                                                       s[p], 0, 0, 0);
    }

    float x[NPASS][4], mx[NPASS];
    bool trig = false;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[p][j] = s[p][j] * scale_log2;  // raw q.k times |scale| log2 e
        if (MASKED && tok0 + 4 * j >= t_end) x[p][j] = -INFINITY;
      }
      mx[p] = fmaxf(fmaxf(x[p][0], x[p][1]), fmaxf(x[p][2], x[p][3]));
      trig |= mx[p] > mrun[p] + kLazyLog2;
    }
    // The reference max of a head is raised (wave-wide) only when a score exceeds it by
    // more than 2^kLazyLog2; acc and l are rescaled then, and acc / l is unchanged.
    if (__any(trig)) {
      float alpha[NPASS];
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        // over the lanes of this head: every GQ-th lane of a row (row rotations by
        // GQ, 2 GQ, ... keep the lane's class mod GQ), then the four rows
        float M = mx[p];
        if constexpr (GQ == 1) M = fmaxf(M, row_ror<1>(M));
        if constexpr (GQ <= 2) M = fmaxf(M, row_ror<2>(M));
        M = fmaxf(M, row_ror<4>(M));
        M = fmaxf(M, row_ror<8>(M));
        M = rows4_max(M);
        const float m_new = fmaxf(mrun[p], M);
        const float m_ref = (m_new > mrun[p] + kLazyLog2) ? m_new : mrun[p];
        alpha[p] = (m_ref == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun[p] - m_ref);
        lrun[p] *= alpha[p];
        mrun[p] = m_ref;
      }
      if constexpr (kPvMfma) {  // the lane's column is one head of each pass
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
#pragma unroll
          for (int e = 0; e < E; ++e) accm[p][e] *= alpha[p];
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float a = quad_bcast(alpha[h / GQ], h % GQ);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= a;
        }
      }
    }
    // weights of this lane's head, packed as bf16 pairs of tokens (g, g+4), (g+8, g+12)
    uint32_t pk[NPASS][2];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const float msub = mrun[p] == -INFINITY ? 0.f : mrun[p];
      float w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = __builtin_amdgcn_exp2f(x[p][j] - msub);
      lrun[p] += (w[0] + w[1]) + (w[2] + w[3]);
      pk[p][0] = pack_bf16x2(w[0], w[1]);
      pk[p][1] = pack_bf16x2(w[2], w[3]);
    }
    if constexpr (kFp8) {
      // V arrives as raw 16-byte chunks (see the kernel's load): vw[2c] / vw[2c + 1] hold the
      // low / high 8 bytes of this lane's chunk c. The lane pair swaps the halves the other
      // lane needs (DPP quad_perm 1,0,3,2), so that vw[i] becomes row g + 4i, own dims.
      const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const bool odd = ln & 1;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < WKV; ++k) {
          const uint32_t lo = vw[2 * c][k], hi = vw[2 * c + 1][k];
          const uint32_t recv =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? lo : hi), 0xB1, 0xF, 0xF, false);
          vw[2 * c][k] = odd ? recv : lo;
          vw[2 * c + 1][k] = odd ? hi : recv;
        }
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + 4 * i >= t_end) {
#pragma unroll
          for (int y = 0; y < WKV; ++y) vw[i][y] = 0u;  // never multiply a dead slot
        }
    }
    uint32_t vb16[4][W32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kFp8) {
#pragma unroll
        for (int y = 0; y < WKV; ++y) {
          vb16[i][2 * y] = fp8x2_to_bf16x2<TKV>(vw[i][y], false);
          vb16[i][2 * y + 1] = fp8x2_to_bf16x2<TKV>(vw[i][y], true);
        }
      } else {
#pragma unroll
        for (int y = 0; y < W32; ++y) vb16[i][y] = vw[i][y];
      }
    }
    if constexpr (kPvMfma) {
      // block e = 2y (low halves) and 2y + 1 (high halves): A = (rows 0, 1), (rows 2, 3) of
      // dim lane_dim(n, e); B = this lane's weights (tokens g, g+4), (g+8, g+12)
#pragma unroll
      for (int y = 0; y < W32; ++y) {
        const uint32_t lo01 = __builtin_amdgcn_perm(vb16[1][y], vb16[0][y], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vb16[1][y], vb16[0][y], 0x07060302u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vb16[3][y], vb16[2][y], 0x05040100u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vb16[3][y], vb16[2][y], 0x07060302u);
        const s16x4_mq alo = __builtin_bit_cast(s16x4_mq, u32x2_t{lo01, lo23});
        const s16x4_mq ahi = __builtin_bit_cast(s16x4_mq, u32x2_t{hi01, hi23});
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          const s16x4_mq bw = __builtin_bit_cast(s16x4_mq, u32x2_t{pk[p][0], pk[p][1]});
          accm[p][2 * y] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bw, accm[p][2 * y], 0, 0, 0);
          accm[p][2 * y + 1] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bw, accm[p][2 * y + 1], 0, 0, 0);
        }
      }
      return;
    }
    // PV on bf16 pairs (tokens 2j', 2j'+1 of this lane's rows), fp32 accumulation
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint32_t pp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pp[h] = quad_bcast(pk[h / GQ][jp], h % GQ);
#pragma unroll
      for (int y = 0; y < W32; ++y) {
        const uint32_t lo = __builtin_amdgcn_perm(vb16[2 * jp + 1][y], vb16[2 * jp][y], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(vb16[2 * jp + 1][y], vb16[2 * jp][y], 0x07060302u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * y] = dot2_bf16(pp[h], lo, acc[h][2 * y]);
          acc[h][2 * y + 1] = dot2_bf16(pp[h], hi, acc[h][2 * y + 1]);
        }
      }
    }
  }
};

}  // namespace gqa
