// Causal GQA prefill on gfx950 with bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// What is computed: out[b][i][h] = softmax_j<=i(scale * q_i . k_j) v_j for the S new
// tokens of every sequence (causal mask: caption of Figure 2 on page
// "解锁GQA性能潜力：从批量大小敏感性到高效优化实践"), query head h reading KV head
// h / G (page "TensorRT对Grouped Query Attention的支持进展", section "技术演进背景"),
// evaluated tile by tile with an online softmax so that no score matrix reaches
// memory and only the output is written (page "TensorRT-LLM与TensorRT核心差异解析",
// section 4.2.1).
//
// Work decomposition: one workgroup (8 waves) per (b, kvh, q-tile). The q-tile holds
// 256 query rows: all G heads of the group x 256/G positions (the G heads are packed
// into one workgroup so that every K/V tile is staged in LDS once and read by all of
// them). Wave w owns 32 rows: one head, 32 consecutive positions. Workgroups are
// issued heaviest (last) q-tile first; blockIdx.x runs over (b, kvh) so all q-tiles
// of one (b, kvh) land on the same XCD and share its L2.
//
// Per 64-key tile and wave (all on-chip):
//   S^T = K Q^T   16 MFMAs; A = K rows from LDS (ds_read_b128, XOR-swizzled rows),
//                 B = Q^T held in registers for the whole kernel.
//   softmax       S^T's C layout gives every lane 32 scores of ONE query, so the row
//                 max / sum are lane-local plus one exchange between the two half-waves;
//                 exp2 with scale*log2(e) folded in; the running max is only raised when
//                 it grows by more than 2^8 (lazy rescale, exact after normalisation).
//   O^T += V^T P^T 16 MFMAs; A = V^T read straight from the key-major V tile with
//                 ds_read_b64_tr_b16 (no transpose pass), B = P^T from registers (bf16).
// K/V tiles stream HBM -> LDS with global_load_lds_dwordx4, double-buffered.
#include <type_traits>

#include "device_common.h"
#include "../../include/gqa.h"

namespace gqa {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

namespace prefill {
constexpr int D = 128;
constexpr int BN = 64;          // keys per tile
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * kWave;
constexpr int ROWB = D * 2;     // bytes per K/V row
constexpr int TILE = BN * ROWB; // 16 KiB
constexpr float kLazy = 8.0f;   // log2 growth tolerated before rescaling O

// Row swizzles (16-byte chunk index XOR): K rows are read 16 at a time at one chunk,
// V rows 4 at a time over 4 chunks (transpose reads).
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

// 16 bytes per lane from a raw buffer straight into LDS (buffer_load_dwordx4 ... lds; LDS
// address M0 + 16 * lane). Written as assembly so that the compiler does not track it: it
// would otherwise treat every later transpose read of LDS as possibly depending on it and
// wait for all loads in flight. The kernel orders the LDS write itself (s_waitcnt vmcnt on
// the issuing wave, then a workgroup barrier) before any wave reads that stage.
__device__ __forceinline__ void buffer_dma16(u32x4_t rsrc, uint32_t voffset, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// Raw buffer descriptor: 48-bit base, stride 0, num_records bytes, gfx9 data format word.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)num_records), 0x00020000u};
}
}  // namespace prefill

// PAGED = false: causal prefill of S new tokens per sequence (positions 0..S-1); K/V tiles
// are read from the new k / v, and the kernel also appends them to the cache.
// PAGED = true: chunked prefill. Sequence b already holds past_lens[b] tokens in the cache
// and its new_lens[b] new tokens (already appended by append_at_kernel) sit at positions
// past .. past+new-1; new row i attends keys 0 .. past+i, all read from the paged cache.
template <int G, bool PAGED>
__global__ __launch_bounds__(prefill::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_causal_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ out, bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ past_lens,
    const int32_t* __restrict__ new_lens, int max_pages, int S, int Hq, int Hkv,
    float scale_log2, int n_qtiles) {
  using namespace prefill;
  constexpr int BMPOS = 256 / G;  // positions per q-tile
  constexpr int PB = 8 / G;       // 32-position blocks per head

  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];  // [stage][K, V]

  const int bkv = blockIdx.x;
  const int b = bkv / Hkv;
  const int kvh = bkv % Hkv;
  const int qt = n_qtiles - 1 - (int)blockIdx.y;
  const int q0 = qt * BMPOS;
  const int w = wave_id();
  const int lane = lane_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hl = w / PB;
  const int h = kvh * G + hl;
  const int qa = q0 + 32 * (w % PB);  // first new row of this wave
  const int my_q = qa + l32;          // the new row this lane's softmax state belongs to

  // p: tokens already cached before this call's rows, n: live new rows (lengths clamped
  // to what the page table row can address)
  int p = 0, n = S;
  if constexpr (PAGED) {
    const int cap = max_pages * 16;
    p = min(max(past_lens[b], 0), cap);
    n = min(max(new_lens[b], 0), min(S, cap - p));
    if (q0 >= n) return;  // the whole workgroup: no live row (before any barrier)
  }
  const int end = p + n;  // keys of the sequence after this call
  const int my_pos = p + my_q;  // absolute position of this lane's query
  const int wave_tiles = qa < n ? (p + min(qa + 31, n - 1)) / BN + 1 : 0;
  const int wg_tiles = (p + min(q0 + BMPOS, n) - 1) / BN + 1;
  const int mask_from = (p + qa) / BN;  // tiles before it are below every row of the wave

  // K and V of (b, kvh) as raw buffers; token t's row starts at byte t * row_stride
  // (PAGED: one buffer per (page, kv head) block, built per load).
  const uint32_t row_stride = (uint32_t)Hkv * ROWB;
  const size_t bkv_off = (size_t)b * S * Hkv * D + (size_t)kvh * D;
  const uint32_t extent = (uint32_t)(S - 1) * row_stride + ROWB;
  const u32x4_t k_rsrc = make_rsrc(k + bkv_off, extent);
  const u32x4_t v_rsrc = make_rsrc(v + bkv_off, extent);

  // Q^T operand: lane holds dims 16s + 8*half .. +7 of query my_q, for s = 0..7. The
  // softmax below takes the row max of the raw scores and applies the scale inside the
  // exponent, which needs scale > 0: a negative scale is moved onto Q (sign flip, exact),
  // and a zero scale is raised to 1e-30 so that masked (-inf) scores still give exp2 = 0
  // (every finite score then maps to exp2(~0) = 1 in fp32, the uniform weights of scale 0).
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sl2 = fmaxf(fabsf(scale_log2), 1e-30f);
  u32x4_t qop[8];
  {
    const bool ok = my_q < n;
    const bf16_t* qrow = q + (((size_t)b * S + (ok ? my_q : 0)) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4_t t = *(const u32x4_t*)(qrow + 16 * s + 8 * half);
      qop[s] = ok ? (t ^ qsign) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  float m_run = -INFINITY;
  float l_half = 0.f;

  // DMA plan of one tile: wave-instruction wi = ii * WAVES + w moves rows 4*(wi%16) ..
  // +3 of K (ii = 0, 1) or V (ii = 2, 3), 16 lanes per row. A lane's byte offset in the
  // buffer is fixed up to the tile base; rows past S - 1 are clamped onto row S - 1.
  static_assert(WAVES * 2 == 16, "two loads move a K tile, two a V tile");
  const uint32_t smem0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&smem[0][0][0];
  uint32_t dma_off[4], dma_last[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = 4 * ((ii & 1) * WAVES + w) + (lane >> 4);
    const int chunk = (lane & 15) ^ (ii >= 2 ? v_swz(r) : k_swz(r));
    dma_off[ii] = (uint32_t)r * row_stride + chunk * 16;
    dma_last[ii] = (uint32_t)(S - 1) * row_stride + chunk * 16;
  }
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(smem0 + w * 1024);
  // PAGED: a load moves 4 consecutive keys, which share one 16-key page. Its first key
  // g0 (clamped onto end - 1) picks the page through the page table; a lane's key is
  // clamped onto end - 1 too (that row exists: keys past the rows of this workgroup are
  // masked, but their V must be finite), and its byte offset in the (page, kv head) block
  // is slot * 256 + the swizzled chunk.
  auto paged_dma = [&](const bf16_t* cache, int t, int ii, uint32_t lds) {
    const int wi2 = (ii & 1) * WAVES + w;
    const int g0 = t * BN + 4 * wi2;
    const int gk = min(g0, end - 1);
    const int page = page_table[(size_t)b * max_pages + (gk >> 4)];
    const int key = min(g0 + (lane >> 4), end - 1);
    const int chunk = (lane & 15) ^ (ii >= 2 ? v_swz(4 * wi2 + (lane >> 4)) : k_swz(4 * wi2 + (lane >> 4)));
    const u32x4_t rsrc = make_rsrc(cache + ((size_t)page * Hkv + kvh) * 16 * D, 16 * ROWB);
    buffer_dma16(rsrc, (uint32_t)((key & 15) * ROWB + chunk * 16), lds);
  };
  auto issue_k = [&](int t, int st) {  // K tile t into stage st
    const uint32_t off = (uint32_t)t * BN * row_stride;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      if constexpr (PAGED)
        paged_dma(k_cache, t, ii, dma_lds + st * 2 * TILE + ii * WAVES * 1024);
      else
        buffer_dma16(k_rsrc, min(dma_off[ii] + off, dma_last[ii]),
                     dma_lds + st * 2 * TILE + ii * WAVES * 1024);
    }
  };
  auto issue_v = [&](int t, int st) {  // V tile t into stage st
    const uint32_t off = (uint32_t)t * BN * row_stride;
#pragma unroll
    for (int ii = 2; ii < 4; ++ii) {
      if constexpr (PAGED)
        paged_dma(v_cache, t, ii, dma_lds + st * 2 * TILE + TILE + (ii & 1) * WAVES * 1024);
      else
        buffer_dma16(v_rsrc, min(dma_off[ii] + off, dma_last[ii]),
                     dma_lds + st * 2 * TILE + TILE + (ii & 1) * WAVES * 1024);
    }
  };

  // Per-lane LDS byte offsets, fixed for the whole kernel (stage, key block and row step
  // are compile-time and become instruction offsets):
  //   K, A operand of step s: row l32, 16-byte chunk (2s + half) ^ (l32 % 16);
  //   V^T, transpose reads: lane (g16, i16) reads row 4*(g16/2) + i16/4 (+16 sp + 8 r) at
  //   chunk 4*mbd + 2*(g16%2) + (i16%4)/2 with the row swizzle 4*(row % 4), i.e.
  //   4*(mbd ^ (i16/4)) + ..., byte (i16%2)*8 of the chunk.
  uint32_t koff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = smem0 + l32 * ROWB + (((2 * s + half) ^ (l32 & 15)) << 4);
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t vlane = smem0 + TILE + (4 * (g16 >> 1) + (i16 >> 2)) * ROWB +
                         (2 * (g16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8;
  uint32_t voff[4];
#pragma unroll
  for (int mbd = 0; mbd < 4; ++mbd) voff[mbd] = vlane + ((mbd ^ (i16 >> 2)) << 6);

  // S^T = K Q^T for the tile in stage ST: two 32-key blocks (16 MFMAs, two chains). The
  // K operands are read PF steps ahead so that LDS latency stays off the MFMA chain
  // (sched_barrier keeps the compiler from sinking the reads next to their use).
  f32x16_t sacc[2];
  auto scores = [&](auto st_tag) {
    constexpr uint32_t SOFF = decltype(st_tag)::value * 2 * TILE;
    constexpr int PF = 3;
    auto kread = [&](int s, int mb) {
      return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
          koff[s] + SOFF + mb * 32 * ROWB);
    };
    u32x4_t ka[PF + 1][2];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      ka[s][0] = kread(s, 0);
      ka[s][1] = kread(s, 1);
    }
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + PF < 8) {
        ka[(s + PF) % (PF + 1)][0] = kread(s + PF, 0);
        ka[(s + PF) % (PF + 1)][1] = kread(s + PF, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, ka[s % (PF + 1)][mb]),
            __builtin_bit_cast(bf16x8_t, qop[s]), sacc[mb], 0, 0, 0);
    }
  };

  // Online softmax of tile kt's scores (raw; scale * log2(e) is applied inside the
  // exponent, so the running max m_run is in scaled log2 units) into P (bf16, the B
  // operand of PV), with the causal mask on the tile that holds the diagonal.
  u32x4_t pop[4];
  auto softmax = [&](int kt, bool diag) {
    if (diag) {
      const int lim = my_pos - kt * BN - 4 * half;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * mb + 8 * (j >> 2) + (j & 3) > lim) sacc[mb][j] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mb][j]);
    {  // the other half-wave holds the other keys of each 8-key group: swap halves
      const u32x2_t r = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                    false, false));
      mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * sl2;
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new > m_run + kLazy) ? m_new : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_use;
    float psum = 0.f;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[sp >> 1][8 * (sp & 1) + i], sl2, -m_use));
        psum += pv[i];
      }
      pop[sp] = u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                        pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    }
    l_half = l_half * alpha + psum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    }
  };

  // O^T += V^T P^T with V from stage ST (16 MFMAs, four chains), transpose reads issued
  // PF MFMAs ahead.
  auto pv = [&](auto st_tag) {
    constexpr uint32_t SOFF = decltype(st_tag)::value * 2 * TILE;
    constexpr int PF = 3;
    auto vread = [&](int i) {  // operand of MFMA i = 4 sp + mbd
      const int sp = i >> 2, mbd = i & 3;
      const uint32_t a0p = voff[mbd] + SOFF + (16 * sp) * ROWB;
      const s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)a0p);
      const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(a0p + 8 * ROWB));
      const u32x2_t a0 = __builtin_bit_cast(u32x2_t, t0);
      const u32x2_t a1 = __builtin_bit_cast(u32x2_t, t1);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    u32x4_t va[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) va[i] = vread(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + PF < 16) va[(i + PF) % (PF + 1)] = vread(i + PF);
      __builtin_amdgcn_sched_barrier(0);
      oacc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, va[i % (PF + 1)]),
          __builtin_bit_cast(bf16x8_t, pop[i >> 2]), oacc[i & 3], 0, 0, 0);
    }
  };

  // Two wave groups in antiphase. Waves 0-3 (group A) and 4-7 (group B) put one wave of
  // each group on every SIMD. Time is cut into phases by workgroup barriers; in each phase
  // one group runs its MFMA phase (PV of tile t, then the scores of tile t+1) while the
  // other runs its softmax phase (VALU), so matrix and vector units of a SIMD work at the
  // same time. Global phase p: group A runs softmax(t) at p = 2t+1 and MFMA(t) at
  // p = 2t+2 (scores(0) at p = 0); group B runs one phase later. Hence K(t) is read in
  // phases 2t, 2t+1 and V(t) in phases 2t+2, 2t+3. Tile t lives in stage t % 2; at every
  // even phase 2u all waves issue the DMA of K(u+1) and V(u), whose stages were last read
  // in phase 2u-1, and wait for it (vmcnt) before the barrier that opens phase 2u+2.
  // Every wave passes 2 * wg_tiles + 2 barriers.
  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  };
  auto even_phase_dma = [&](int u, auto par_tag) {  // u % 2 == par
    constexpr int PAR = decltype(par_tag)::value;
    if (u + 1 < wg_tiles) issue_k(u + 1, PAR ^ 1);
    if (u < wg_tiles) issue_v(u, PAR);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // tile t (parity PAR) for a wave of group A: softmax at phase 2t+1, MFMA at 2t+2
  auto tile_a = [&](int t, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    bar();  // phase 2t+1
    if (t < wave_tiles) softmax(t, t >= mask_from);
    wait_vmcnt<0>();
    bar();  // phase 2t+2
    even_phase_dma(t + 1, std::integral_constant<int, PAR ^ 1>{});
    if (t < wave_tiles) pv(par_tag);
    if (t + 1 < wave_tiles) scores(std::integral_constant<int, PAR ^ 1>{});
  };
  // tile t for a wave of group B: softmax at phase 2t+2, MFMA at 2t+3
  auto tile_b = [&](int t, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    wait_vmcnt<0>();
    bar();  // phase 2t+2
    even_phase_dma(t + 1, std::integral_constant<int, PAR ^ 1>{});
    if (t < wave_tiles) softmax(t, t >= mask_from);
    bar();  // phase 2t+3
    if (t < wave_tiles) pv(par_tag);
    if (t + 1 < wave_tiles) scores(std::integral_constant<int, PAR ^ 1>{});
  };

  issue_k(0, 0);
  if constexpr (!PAGED) {
  // KV append: this workgroup copies the new K/V rows of its own positions
  // [q0, q0 + BMPOS) of KV head kvh into their cache slots (slot pos % 16 of page
  // page_table[b][pos / 16]); every position of every (b, kvh) is owned by exactly one
  // workgroup. The rows were just requested by the first tile's DMA, so they come from L2.
  {
    const int nrows = min(BMPOS, S - q0);
    for (int idx = (int)threadIdx.x; idx < nrows * 32; idx += THREADS) {
      const int is_v = idx >= nrows * 16;
      const int rem = idx - is_v * nrows * 16;
      const int pos = q0 + (rem >> 4), c = rem & 15;
      const int page = page_table[(size_t)b * max_pages + (pos >> 4)];
      const u32x4_t x =
          *(const u32x4_t*)((is_v ? v : k) + ((size_t)(b * S + pos) * Hkv + kvh) * D + c * 8);
      *(u32x4_t*)((is_v ? v_cache : k_cache) + (((size_t)page * Hkv + kvh) * 16 + (pos & 15)) * D +
                  c * 8) = x;
    }
  }
  }
  wait_vmcnt<0>();  // K(0) has landed (and the append's stores have completed)
  bar();  // phase 0
  even_phase_dma(0, P0{});
  if (w < 4) {
    if (wave_tiles > 0) scores(P0{});
    for (int t = 0; t < wg_tiles; t += 2) {
      tile_a(t, P0{});
      if (t + 1 < wg_tiles) tile_a(t + 1, P1{});
    }
    bar();
  } else {
    bar();  // phase 1
    if (wave_tiles > 0) scores(P0{});
    for (int t = 0; t < wg_tiles; t += 2) {
      tile_b(t, P0{});
      if (t + 1 < wg_tiles) tile_b(t + 1, P1{});
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue: O = O^T / l, bf16, 4 consecutive dims per store ----
  if (wave_tiles == 0 || my_q >= n) return;
  const float l_tot = l_half + __shfl_xor(l_half, 32);
  const float inv = 1.0f / l_tot;
  bf16_t* orow = out + (((size_t)b * S + my_q) * Hq + h) * D;
#pragma unroll
  for (int mbd = 0; mbd < 4; ++mbd)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int dim = 32 * mbd + 8 * jq + 4 * half;
      const u32x2_t pk = {pack_bf16x2(oacc[mbd][4 * jq + 0] * inv, oacc[mbd][4 * jq + 1] * inv),
                          pack_bf16x2(oacc[mbd][4 * jq + 2] * inv, oacc[mbd][4 * jq + 3] * inv)};
      *(u32x2_t*)(orow + dim) = pk;
    }
}

// Chunked prefill, step 1: new[b][i] (i < new_lens[b]) -> cache slot of position
// past_lens[b] + i; one thread per 16-byte chunk of a (row, kv head), K and V. Lengths are
// clamped exactly as in the attention kernel.
__global__ __launch_bounds__(256) void append_at_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, bf16_t* __restrict__ k_cache,
    bf16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ past_lens, const int32_t* __restrict__ new_lens, int S, int Hkv,
    int max_pages) {
  using namespace prefill;
  const int b = blockIdx.y;
  const int cap = max_pages * 16;
  const int p = min(max(past_lens[b], 0), cap);
  const int n = min(max(new_lens[b], 0), min(S, cap - p));
  const int idx = blockIdx.x * 256 + threadIdx.x;  // over [S][Hkv][16 chunks]
  const int i = idx / (Hkv * 16);
  if (i >= n) return;
  const int kvh = (idx / 16) % Hkv, c = idx & 15;
  const int pos = p + i;
  const int page = page_table[(size_t)b * max_pages + (pos >> 4)];
  const size_t src = ((size_t)(b * S + i) * Hkv + kvh) * D + c * 8;
  const size_t dst = (((size_t)page * Hkv + kvh) * 16 + (pos & 15)) * D + c * 8;
  *(u32x4_t*)(k_cache + dst) = *(const u32x4_t*)(k + src);
  *(u32x4_t*)(v_cache + dst) = *(const u32x4_t*)(v + src);
}

template <int G, bool PAGED>
static int launch_g(const void* q, const void* k, const void* v, void* out, void* k_cache,
                    void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                    const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv,
                    float scale, hipStream_t s) {
  constexpr int BMPOS = 256 / G;
  const int n_qtiles = (S + BMPOS - 1) / BMPOS;
  dim3 grid((unsigned)(B * Hkv), (unsigned)n_qtiles);
  hipLaunchKernelGGL((prefill_causal_kernel<G, PAGED>), grid, dim3(prefill::THREADS), 0, s,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)out,
                     (bf16_t*)k_cache, (bf16_t*)v_cache, page_table, past_lens, new_lens,
                     max_pages, S, Hq, Hkv, scale * kLog2e, n_qtiles);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <bool PAGED>
static int launch_any(const void* q, const void* k, const void* v, void* out, void* k_cache,
                      void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                      const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv, int D,
                      float scale, hipStream_t s) {
  if (D != prefill::D) return GQA_ERR_UNSUPPORTED;
  switch (Hq / Hkv) {
    case 1: return launch_g<1, PAGED>(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens, max_pages, B, S, Hq, Hkv, scale, s);
    case 2: return launch_g<2, PAGED>(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens, max_pages, B, S, Hq, Hkv, scale, s);
    case 4: return launch_g<4, PAGED>(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens, max_pages, B, S, Hq, Hkv, scale, s);
    case 8: return launch_g<8, PAGED>(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens, max_pages, B, S, Hq, Hkv, scale, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_prefill(const void* q, const void* k, const void* v, void* out, void* k_cache,
                   void* v_cache, const int32_t* page_table, int max_pages, int B, int S, int Hq,
                   int Hkv, int D, float scale, hipStream_t s) {
  return launch_any<false>(q, k, v, out, k_cache, v_cache, page_table, nullptr, nullptr,
                           max_pages, B, S, Hq, Hkv, D, scale, s);
}

int launch_prefill_paged(const void* q, const void* k, const void* v, void* out, void* k_cache,
                         void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                         const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv,
                         int D, float scale, hipStream_t s) {
  if (D != prefill::D) return GQA_ERR_UNSUPPORTED;
  const int chunks = S * Hkv * 16;
  hipLaunchKernelGGL(append_at_kernel, dim3((unsigned)((chunks + 255) / 256), (unsigned)B),
                     dim3(256), 0, s, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)k_cache,
                     (bf16_t*)v_cache, page_table, past_lens, new_lens, S, Hkv, max_pages);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_LAUNCH;
  return launch_any<true>(q, k, v, out, k_cache, v_cache, page_table, past_lens, new_lens,
                          max_pages, B, S, Hq, Hkv, D, scale, s);
}

}  // namespace gqa
