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
// Work decomposition: the unit of work (an item) is a (b, kvh, q-tile). The q-tile holds
// 256 query rows: all G heads of the group x 256/G positions (the G heads are packed
// into one workgroup so that every K/V tile is staged in LDS once and read by all of
// them). Wave w of the 8 owns 32 rows: one head, 32 consecutive positions. The kernel is
// persistent: one workgroup per compute unit serves one (b, kvh) and walks a list of its
// q-tiles (schedule at the kernel), so that a workgroup's start-up (Q rows, first key
// tile) and its stores overlap work instead of leaving the compute unit idle between
// workgroups.
//
// Per 64-key tile and wave (all on-chip):
//   S^T = K Q^T   16 MFMAs; A = K rows from LDS (ds_read_b128, XOR-swizzled rows),
//                 B = Q^T held in registers for the whole item (read from LDS, where
//                 the previous item fetched it).
//   softmax       S^T's C layout gives every lane 32 scores of ONE query, so the row
//                 max / sum are lane-local plus one exchange between the two half-waves;
//                 exp2 with scale*log2(e) folded in; the running max is only raised when
//                 it grows by more than 2^8 (lazy rescale, exact after normalisation).
//   O^T += V^T P^T 16 MFMAs; A = V^T read straight from the key-major V tile with
//                 ds_read_b64_tr_b16 (no transpose pass), B = P^T from registers (bf16).
// K/V tiles stream HBM -> LDS with global_load_lds_dwordx4, double-buffered.
#include <algorithm>
#include <atomic>
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
constexpr int kNt = 2;          // cache-policy bit of the buffer builtins: streaming (nt)

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

// The same with the streaming (nt) hint, for data read once (the Q rows): it leaves the L2 to
// the K/V tiles that the other q-tiles of the pair read again. Used for G <= 2, with the
// output and KV-append stores streamed too: there it measured faster (G = 1: 182 -> 175 us at
// B=4, S=2048, Hq=32). For G = 4 (B=4, S=2048, Hq=32, Hkv=8) it cut the HBM traffic from 1.30x
// to 1.10x of the algorithmic bytes but took 2-3% longer, so G >= 4 keeps ordinary loads and
// stores.
__device__ __forceinline__ void buffer_dma16_nt(u32x4_t rsrc, uint32_t voffset, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// 4 bytes per lane from a raw buffer into LDS (LDS address M0 + 4 * lane); same ordering
// rules as buffer_dma16.
__device__ __forceinline__ void buffer_dma4(u32x4_t rsrc, uint32_t voffset, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// The lane index, computed afresh (v_mbcnt) where it is used: the asm statement cannot be
// hoisted, so the compiler neither keeps it nor values derived from it live across loops.
__device__ __forceinline__ int fresh_lane() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
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
//
// Persistent schedule: workgroup g serves the (b, kv head) pair c = g % nbkv and walks a
// list of its q-tiles (items). With A = rows_per_round workgroups per pair, round r gives
// workgroup row a = g / nbkv the q-tile of rank r * A + a (r even) or r * A + A - 1 - a
// (r odd), rank 0 being the last, heaviest q-tile: the causal triangle is dealt out in a
// snake so that every workgroup gets a near-equal number of key tiles, and all q-tiles of
// one pair run on the XCD of its workgroups (workgroup g runs on XCD g % 8, and c % 8 ==
// g % 8 when 8 divides nbkv) and share its L2. Between two items the workgroup does not
// drain: the next item's Q rows are fetched into LDS while the current item still runs,
// and an item's output is stored (from the Q rows' LDS) after the next item has started.
template <int G, bool PAGED>
__global__ __launch_bounds__(prefill::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_causal_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ out, bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ past_lens,
    const int32_t* __restrict__ new_lens, int max_pages, int S, int Hq, int Hkv,
    float scale_log2, int n_qtiles, int nbkv, int rows_per_round) {
  using namespace prefill;
  constexpr int BMPOS = 256 / G;  // positions per q-tile
  constexpr int PB = 8 / G;       // 32-position blocks per head
  constexpr bool kStream = G <= 2;  // streaming hint on Q rows, output and KV-append stores

  // LDS: [stage][K, V] tiles (64 KiB); K tile 0, loaded once (16 KiB: every item of the
  // workgroup has the same (b, kv head), hence the same first key tile); the Q rows of
  // the next item, 8 KiB per wave (64 KiB); the current item's page ids, 256 bytes per wave
  // (causal prefill: used by the KV append).
  constexpr uint32_t K0_OFF = 2 * 2 * TILE;
  constexpr uint32_t Q_OFF = K0_OFF + TILE;
  constexpr uint32_t PT_OFF = Q_OFF + WAVES * 32 * ROWB;
  __shared__ __attribute__((aligned(16))) char smem[PT_OFF + WAVES * 256];

  const int bkv = (int)blockIdx.x % nbkv;
  const int arow = (int)blockIdx.x / nbkv;
  const int b = bkv / Hkv;
  const int kvh = bkv % Hkv;
  const int w = wave_id();
  const int hl = w / PB;
  const int h = kvh * G + hl;

  // p: tokens already cached before this call's rows, n: live new rows (lengths clamped
  // to what the page table row can address)
  int p = 0, n = S;
  if constexpr (PAGED) {
    const int cap = max_pages * 16;
    p = min(max(past_lens[b], 0), cap);
    n = min(max(new_lens[b], 0), min(S, cap - p));
  }
  const int end = p + n;  // keys of the sequence after this call
  // q-tile of round r (-1 past the last round), and the next round after r whose q-tile
  // holds a live row (-1 if none): a short chunk leaves the heaviest q-tiles empty
  auto qt_of = [&](int r) {
    const int rank = r * rows_per_round + ((r & 1) ? rows_per_round - 1 - arow : arow);
    return rank < n_qtiles ? n_qtiles - 1 - rank : -1;
  };
  auto next_round = [&](int r) {
    for (++r;; ++r) {
      const int qt = qt_of(r);
      if (qt < 0) return -1;
      if (qt * BMPOS < n) return r;
    }
  };
  int r = next_round(-1);
  if (r < 0) return;  // the whole workgroup: no live q-tile (before any barrier)

  // K and V of (b, kvh) as raw buffers; token t's row starts at byte t * row_stride
  // (PAGED: one buffer per (page, kv head) block, built per load). Q rows of head h:
  // row i at byte i * q_stride.
  const uint32_t row_stride = (uint32_t)Hkv * ROWB;
  const size_t bkv_off = (size_t)b * S * Hkv * D + (size_t)kvh * D;
  const uint32_t extent = (uint32_t)(S - 1) * row_stride + ROWB;
  const u32x4_t k_rsrc = make_rsrc(k + bkv_off, extent);
  const u32x4_t v_rsrc = make_rsrc(v + bkv_off, extent);
  const uint32_t q_stride = (uint32_t)Hq * ROWB;

  // The softmax below takes the row max of the raw scores and applies the scale inside the
  // exponent, which needs scale > 0: a negative scale is moved onto Q (sign flip, exact),
  // and a zero scale is raised to 1e-30 so that masked (-inf) scores still give exp2 = 0
  // (every finite score then maps to exp2(~0) = 1 in fp32, the uniform weights of scale 0).
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sl2 = fmaxf(fabsf(scale_log2), 1e-30f);

  // Item state (set per q-tile): first position q0, this wave's first row qa (a lane's
  // query row is qa + lane % 32), the key tiles of the wave / workgroup and the first tile
  // that needs the causal mask for this wave. Per-lane values are derived from fresh_lane()
  // where they are used.
  int q0 = 0, qa = 0, wave_tiles = 0, wg_tiles = 0, mask_from = 0;
  // The next item's Q rows are requested at even phase 2 * u_pf (with V(u_pf)), into this
  // wave's own LDS rows, which it read at phase 0.
  bool has_next = false;
  int u_pf = 1, qa_next = 0;

  u32x4_t qop[8];
  f32x16_t oacc[4];
  float m_run = -INFINITY;
  float l_half = 0.f;

  // DMA plan of one tile: wave-instruction wi = ii * WAVES + w moves rows 4*(wi%16) ..
  // +3 of K (ii = 0, 1) or V (ii = 2, 3), 16 lanes per row. A lane's byte offset in the
  // buffer is fixed up to the tile base; rows past S - 1 are clamped onto row S - 1.
  static_assert(WAVES * 2 == 16, "two loads move a K tile, two a V tile");
  const uint32_t smem0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&smem[0];
  // (Computed per tile from a lane index the compiler cannot see through: offsets kept in
  // registers for the whole kernel get spilled, and reloading a spilled value waits for every
  // load in flight, the tile DMA included.)
  struct DmaLane {
    uint32_t off[4], last[4];
  };
  auto dma_lane = [&]() {
    const int ln = fresh_lane();
    DmaLane d;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int row = 4 * ((ii & 1) * WAVES + w) + (ln >> 4);
      const int chunk = (ln & 15) ^ (ii >= 2 ? v_swz(row) : k_swz(row));
      d.off[ii] = (uint32_t)row * row_stride + chunk * 16;
      d.last[ii] = (uint32_t)(S - 1) * row_stride + chunk * 16;
    }
    return d;
  };
  const uint32_t dma_lds = __builtin_amdgcn_readfirstlane(smem0 + w * 1024);
  // PAGED: a load moves 4 consecutive keys, which share one 16-key page. Its first key
  // g0 (clamped onto end - 1) picks the page through the page table; a lane's key is
  // clamped onto end - 1 too (that row exists: keys past the rows of this workgroup are
  // masked, but their V must be finite), and its byte offset in the (page, kv head) block
  // is slot * 256 + the swizzled chunk.
  auto paged_dma = [&](const bf16_t* cache, int t, int ii, uint32_t lds) {
    const int ln = fresh_lane();
    const int wi2 = (ii & 1) * WAVES + w;
    const int g0 = t * BN + 4 * wi2;
    const int gk = min(g0, end - 1);
    const int page = page_table[(size_t)b * max_pages + (gk >> 4)];
    const int key = min(g0 + (ln >> 4), end - 1);
    const int chunk = (ln & 15) ^ (ii >= 2 ? v_swz(4 * wi2 + (ln >> 4)) : k_swz(4 * wi2 + (ln >> 4)));
    const u32x4_t rsrc = make_rsrc(cache + ((size_t)page * Hkv + kvh) * 16 * D, 16 * ROWB);
    buffer_dma16(rsrc, (uint32_t)((key & 15) * ROWB + chunk * 16), lds);
  };
  // (The LDS base goes through an empty asm statement so that the compiler adds the stage
  // offsets per call instead of keeping every stage's address in its own scalar register.)
  auto issue_k = [&](int t, int st, const DmaLane& d) {  // K tile t into stage st
    const uint32_t off = (uint32_t)t * BN * row_stride;
    uint32_t lds = dma_lds;
    asm volatile("" : "+s"(lds));
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      if constexpr (PAGED)
        paged_dma(k_cache, t, ii, lds + st * 2 * TILE + ii * WAVES * 1024);
      else
        buffer_dma16(k_rsrc, min(d.off[ii] + off, d.last[ii]), lds + st * 2 * TILE + ii * WAVES * 1024);
    }
  };
  auto issue_v = [&](int t, int st, const DmaLane& d) {  // V tile t into stage st
    const uint32_t off = (uint32_t)t * BN * row_stride;
    uint32_t lds = dma_lds;
    asm volatile("" : "+s"(lds));
#pragma unroll
    for (int ii = 2; ii < 4; ++ii) {
      if constexpr (PAGED)
        paged_dma(v_cache, t, ii, lds + st * 2 * TILE + TILE + (ii & 1) * WAVES * 1024);
      else
        buffer_dma16(v_rsrc, min(d.off[ii] + off, d.last[ii]),
                     lds + st * 2 * TILE + TILE + (ii & 1) * WAVES * 1024);
    }
  };

  // Q rows qa .. qa + 31 of an item into this wave's 8 KiB of LDS, 4 rows (16 lanes each) per
  // load: row i of the wave goes to LDS row i, its 16-byte chunks XOR-swizzled by i % 16 like
  // the K rows. Rows past S - 1 are clamped onto row S - 1 (their queries are not live).
  const uint32_t qbuf = __builtin_amdgcn_readfirstlane(smem0 + Q_OFF + w * 32 * ROWB);
  // (The lane index is passed through an empty asm statement so that the compiler computes
  // the offsets per call instead of keeping them live through the kernel.)
  auto fetch_q = [&](int qa_item) {
    const int ln = fresh_lane();
    uint32_t lds = qbuf;
    asm volatile("" : "+s"(lds));
    const u32x4_t rsrc = make_rsrc(q + ((size_t)b * S * Hq + h) * D, (uint32_t)(S - 1) * q_stride + ROWB);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ri = 4 * j + (ln >> 4);
      const int row = min(qa_item + ri, S - 1);
      if constexpr (kStream)
        buffer_dma16_nt(rsrc, (uint32_t)row * q_stride + (((ln & 15) ^ (ri & 15)) << 4),
                        lds + j * 1024);
      else
        buffer_dma16(rsrc, (uint32_t)row * q_stride + (((ln & 15) ^ (ri & 15)) << 4),
                     lds + j * 1024);
    }
  };

  // Causal prefill: page ids of the current item's positions, entries (q0 / 16) + lane of
  // the page-table row (clamped to the row), into this wave's 256 bytes of LDS.
  auto fetch_pages = [&]() {
    const int ln = fresh_lane();
    uint32_t lds = __builtin_amdgcn_readfirstlane(smem0 + PT_OFF + w * 256);
    asm volatile("" : "+s"(lds));
    const u32x4_t rsrc = make_rsrc(page_table + (size_t)b * max_pages, (uint32_t)max_pages * 4);
    buffer_dma4(rsrc, (uint32_t)min((q0 >> 4) + ln, max_pages - 1) * 4, lds);
  };

  // Per-lane LDS byte offsets (stage, key block and row step are compile-time and become
  // instruction offsets):
  //   K, A operand of step s: row l32, 16-byte chunk (2s + half) ^ (l32 % 16);
  //   V^T, transpose reads: lane (g16, i16) reads row 4*(g16/2) + i16/4 (+16 sp + 8 r) at
  //   chunk 4*mbd + 2*(g16%2) + (i16%4)/2 with the row swizzle 4*(row % 4), i.e.
  //   4*(mbd ^ (i16/4)) + ..., byte (i16%2)*8 of the chunk.
  // These are recomputed at the start of every item (the DMA offsets for every tile) from a
  // lane index the compiler cannot see through: values kept live around the item loop would
  // not fit in the register file next to the tile loop's.
  uint32_t koff[8], voff[4];
  auto set_lane_offsets = [&]() {
    const int ln = fresh_lane();
    const int l32x = ln & 31, hx = ln >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) koff[s] = smem0 + l32x * ROWB + (((2 * s + hx) ^ (l32x & 15)) << 4);
    const int g16 = ln >> 4;
    const int i16 = ln & 15;
    const uint32_t vlane = smem0 + TILE + (4 * (g16 >> 1) + (i16 >> 2)) * ROWB +
                           (2 * (g16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8;
#pragma unroll
    for (int mbd = 0; mbd < 4; ++mbd) voff[mbd] = vlane + ((mbd ^ (i16 >> 2)) << 6);
  };

  // S^T = K Q^T for the tile in stage ST: two 32-key blocks (16 MFMAs, two chains). The
  // K operands are read PF steps ahead so that LDS latency stays off the MFMA chain
  // (sched_barrier keeps the compiler from sinking the reads next to their use).
  f32x16_t sacc[2];
  // K(0)'s buffer lies beyond the 16-bit offset field of the LDS reads: its base is added per
  // read from a register the compiler may not hoist (keeping 8 more addresses live through
  // the whole kernel would spill).
  auto scores = [&](auto st_tag, auto&& hook) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr uint32_t SOFF = ST == 2 ? 0 : ST * 2 * TILE;
    uint32_t base = 0;
    if constexpr (ST == 2) {
      base = K0_OFF;
      asm volatile("" : "+v"(base));
    }
    constexpr int PF = 3;
    auto kread = [&](int s, int mb) {
      return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
          koff[s] + base + SOFF + mb * 32 * ROWB);
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
      hook(s);
    }
  };

  // Online softmax of tile kt's scores (raw; scale * log2(e) is applied inside the
  // exponent, so the running max m_run is in scaled log2 units) into P (bf16, the B
  // operand of PV), with the causal mask on the tile that holds the diagonal.
  u32x4_t pop[4];
  auto softmax = [&](int kt, bool diag) {
    if (diag) {
      const int ln = fresh_lane();
      const int lim = p + qa + (ln & 31) - kt * BN - 4 * (ln >> 5);
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

  // One MFMA phase with both halves: PV of tile t (V from the stage of pv_tag) and the scores
  // of tile t+1 (K from the stage of sc_tag), their MFMAs interleaved one for one. The PV operands come from
  // transpose reads, which the LDS serves at about half the rate of the score loop's b128
  // reads; four waves running PV alone outrun the LDS, the mixed stream does not.
  auto pv_scores = [&](auto pv_tag, auto sc_tag) {
    constexpr uint32_t VOFF = decltype(pv_tag)::value * 2 * TILE;
    constexpr uint32_t KOFF = decltype(sc_tag)::value * 2 * TILE;
    constexpr int PF = 2;
    auto vread = [&](int i) {  // operand of PV MFMA i = 4 sp + mbd
      const int sp = i >> 2, mbd = i & 3;
      const uint32_t a0p = voff[mbd] + VOFF + (16 * sp) * ROWB;
      const s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)a0p);
      const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(a0p + 8 * ROWB));
      const u32x2_t a0 = __builtin_bit_cast(u32x2_t, t0);
      const u32x2_t a1 = __builtin_bit_cast(u32x2_t, t1);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    auto kread = [&](int i) {  // operand of score MFMA i = 2 s + mb
      return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
          koff[i >> 1] + KOFF + (i & 1) * 32 * ROWB);
    };
    u32x4_t va[PF + 1], ka[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      va[i] = vread(i);
      ka[i] = kread(i);
    }
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + PF < 16) {
        va[(i + PF) % (PF + 1)] = vread(i + PF);
        ka[(i + PF) % (PF + 1)] = kread(i + PF);
      }
      __builtin_amdgcn_sched_barrier(0);
      oacc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, va[i % (PF + 1)]),
          __builtin_bit_cast(bf16x8_t, pop[i >> 2]), oacc[i & 3], 0, 0, 0);
      sacc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, ka[i % (PF + 1)]),
          __builtin_bit_cast(bf16x8_t, qop[i >> 1]), sacc[i & 1], 0, 0, 0);
    }
  };
  // PV(t) and scores(t+1) of this wave. On the wave's last tile the scores half runs too (on
  // whatever stage (t+1) % 2 holds; softmax never reads them): one code path for the phase
  // keeps the register allocation of the loop within the register file.
  auto mfma_phase = [&](int t, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    if (t < wave_tiles) pv_scores(par_tag, std::integral_constant<int, PAR ^ 1>{});
  };

  // Two wave groups in antiphase. Waves 0-3 (group A) and 4-7 (group B) put one wave of
  // each group on every SIMD. Time is cut into phases by workgroup barriers; in each phase
  // one group runs its MFMA phase (PV of tile t interleaved with the scores of tile t+1)
  // while the other runs its softmax phase (VALU), so matrix and vector units of a SIMD work
  // at the same time. Global phase p of an item: group A runs softmax(t) at p = 2t+1 and MFMA(t)
  // at p = 2t+2 (scores(0) at p = 0); group B runs one phase later. Hence K(t) is read in
  // phases 2t, 2t+1 and V(t) in phases 2t+2, 2t+3. Tile t >= 1 lives in stage t % 2 (K(0)
  // in its own buffer); in every even phase 2u all waves issue the DMA of K(u+1) and V(u),
  // whose stages were last read in phase 2u-1 (group A at the start of its MFMA phase, group
  // B after its softmax, so that the two halves do not queue up together), and wait for it
  // (vmcnt) before the barrier that opens phase 2u+2. At phase 2 * u_pf the waves also request the next item's Q rows
  // (8 loads per wave) and, for the causal prefill, the item's page ids (1 load), issued
  // after V(u_pf), so the wait before phase 2 * u_pf + 2 leaves those in flight: loads
  // complete in issue order. Every wave passes 2 * wg_tiles + 2 barriers per item.
  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  };
  auto even_phase_dma = [&](int u, auto par_tag) {  // u % 2 == par
    constexpr int PAR = decltype(par_tag)::value;
    DmaLane d{};
    if constexpr (!PAGED) d = dma_lane();
    if (u + 1 < wg_tiles) issue_k(u + 1, PAR ^ 1, d);
    if (u < wg_tiles) issue_v(u, PAR, d);
    if (u == u_pf) {
      if (has_next) fetch_q(qa_next);
      if constexpr (!PAGED) fetch_pages();
    }
  };
  // Before the barrier that opens phase 2t+2: the tile loads of phase 2t must have landed;
  // at t == u_pf the loads issued after them (the next item's Q rows, the page ids) may not.
  auto wait_dma = [&](int t) {
    if (t == u_pf) {
      if (has_next) {
        if constexpr (PAGED) wait_vmcnt<8>(); else wait_vmcnt<9>();
      } else {
        if constexpr (PAGED) wait_vmcnt<0>(); else wait_vmcnt<1>();
      }
    } else {
      wait_vmcnt<0>();
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using PK0 = std::integral_constant<int, 2>;  // K(0)'s own buffer
  // tile t (parity PAR) for a wave of group A: softmax at phase 2t+1, MFMA at 2t+2
  auto tile_a = [&](int t, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    bar();  // phase 2t+1
    if (t < wave_tiles) softmax(t, t >= mask_from);
    wait_dma(t);
    bar();  // phase 2t+2
    even_phase_dma(t + 1, std::integral_constant<int, PAR ^ 1>{});
    mfma_phase(t, par_tag);
  };
  // tile t for a wave of group B: softmax at phase 2t+2, MFMA at 2t+3
  auto tile_b = [&](int t, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    wait_dma(t);
    bar();  // phase 2t+2
    if (t < wave_tiles) softmax(t, t >= mask_from);
    even_phase_dma(t + 1, std::integral_constant<int, PAR ^ 1>{});
    bar();  // phase 2t+3
    mfma_phase(t, par_tag);
  };

  // KV append (causal prefill only): a workgroup copies the new K/V rows of the positions
  // [q0i, q0i + BMPOS) of an item it finished, for KV head kvh, into their cache slots (slot
  // pos % 16 of page page_table[b][pos / 16]); every position of every (b, kvh) belongs to
  // exactly one item. With G = 1 the rows are read again from k / v (they were streamed as
  // the item's last K/V tiles, so the reads mostly hit L2); eight 16-byte chunks per thread
  // are loaded before any is stored.
  auto append_rows = [&](int q0i, int tid, int nthreads) {
    asm volatile("" : "+v"(tid));
    const int nrows = min(BMPOS, S - q0i);
    const int total = nrows * 32;  // 16-byte chunks: K then V, 16 per row
    for (int base = 0; base < total; base += 8 * nthreads) {
      u32x4_t x[8];
      bf16_t* dst[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = min(base + u * nthreads + tid, total - 1);
        const int is_v = idx >= nrows * 16;
        const int rem = idx - is_v * nrows * 16;
        const int pos = q0i + (rem >> 4), c = rem & 15;
        const int page = page_table[(size_t)b * max_pages + (pos >> 4)];
        x[u] = *(const u32x4_t*)((is_v ? v : k) + ((size_t)(b * S + pos) * Hkv + kvh) * D + c * 8);
        dst[u] = (is_v ? v_cache : k_cache) + (((size_t)page * Hkv + kvh) * 16 + (pos & 15)) * D + c * 8;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (base + u * nthreads + tid < total) *(u32x4_t*)dst[u] = x[u];
    }
  };
  // With G >= 2 an item's positions lie in its last one or two key tiles, which are still in
  // LDS when group A has finished the item (K(T-1), V(T-1) in stage (T-1) % 2, K(T-2) and
  // V(T-2) in the other stage or, for tile 0, K(0)'s buffer; nothing is loaded over them
  // before the next item starts), and the page ids were fetched into LDS: the append is LDS
  // reads and global stores only.
  // q0 is a multiple of 16 (BMPOS >= 32), so thread tid of group A always copies 16-byte chunk
  // c = tid % 16 of page slot tid / 16: row block j (rows 16 j .. 16 j + 15 of the item) is
  // page-table entry (q0 / 16) + j, tile (q0 + 16 j) / 64, and the row's swizzle depends on the
  // slot alone. All LDS reads are issued before the first store.
  auto append_from_lds = [&]() {
    constexpr int NJ = BMPOS / 16;  // row blocks of an item
    const int tid = fresh_lane() + kWave * w;  // group A: 256 threads
    const int slot = tid >> 4, c = tid & 15;
    const int nrows = min(BMPOS, S - q0);
    const uint32_t kx = (uint32_t)((c ^ k_swz(slot)) << 4), vx = (uint32_t)((c ^ v_swz(slot)) << 4);
    u32x4_t xk[NJ], xv[NJ];
    int page[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int t = (q0 + 16 * j) / BN;
      const uint32_t row = (uint32_t)((q0 + 16 * j) % BN + slot) * ROWB;
      const uint32_t ktile = t == 0 ? K0_OFF : (uint32_t)(t & 1) * 2 * TILE;
      const uint32_t vtile = (uint32_t)(t & 1) * 2 * TILE + TILE;
      xk[j] = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(smem0 + ktile + row + kx);
      xv[j] = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(smem0 + vtile + row + vx);
      page[j] = *(const __attribute__((address_space(3))) int*)(uintptr_t)(smem0 + PT_OFF + w * 256 + j * 4);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (16 * j + slot < nrows) {
        const size_t off = (((size_t)page[j] * Hkv + kvh) * 16 + slot) * D + c * 8;
        if constexpr (kStream) {
          __builtin_nontemporal_store(xk[j], (u32x4_t*)(k_cache + off));
          __builtin_nontemporal_store(xv[j], (u32x4_t*)(v_cache + off));
        } else {
          *(u32x4_t*)(k_cache + off) = xk[j];
          *(u32x4_t*)(v_cache + off) = xv[j];
        }
      }
    }
  };

  // Rows 4i .. 4i+3 of a staged output tile to the output (rows of head h as a raw buffer, row
  // i at byte i * Hq * ROWB; rows past the live ones get an offset beyond the buffer and the
  // hardware drops their stores)
  auto store_rows = [&](uint32_t sbase, int qa_e, int i) {
    const int ln = fresh_lane();
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        out + ((size_t)b * S * Hq + h) * D, 0, (int)((uint32_t)(S - 1) * q_stride + ROWB), 0x00020000);
    const int rr = 4 * i + (ln >> 4), c = ln & 15;
    const u32x4_t x = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
        sbase + rr * ROWB + ((c ^ (rr & 15)) << 4));
    const int row = qa_e + rr;
    const uint32_t off = row < n ? (uint32_t)row * q_stride + c * 16 : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(x, ors, (int)off, 0, kStream ? kNt : 0);
  };
  // Output of one wave's 32 rows (O = O^T / l, bf16). The MFMA layout gives a lane 4
  // consecutive dims of one row, so the tile is first written to 8 KiB of LDS at sbase (16-byte
  // chunks XOR-swizzled by row % 16) and read back as whole rows, 16 lanes per 256-byte row:
  // each global store then writes four complete rows instead of 16 bytes of each of 32 rows.
  // With qa_e < 0 the tile is only staged (stored later with store_rows).
  // (l_tot: this lane's partial row sum plus that of the lane 32 away, which holds the row's
  // other keys; a VALU exchange, so that the LDS traffic of the other wave group's MFMA phase
  // does not delay it)
  auto row_total = [&]() {
    const u32x2_t r = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(l_half), __float_as_uint(l_half),
                                                  false, false));
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  auto store_output = [&](uint32_t sbase, int qa_e) {
    const int ln = fresh_lane();
    const int rw = ln & 31, hf = ln >> 5;
    const float l_tot = row_total();
    const float inv = 1.0f / l_tot;  // not finite on rows that are not stored
#pragma unroll
    for (int mbd = 0; mbd < 4; ++mbd)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2_t pk = {pack_bf16x2(oacc[mbd][4 * jq + 0] * inv, oacc[mbd][4 * jq + 1] * inv),
                            pack_bf16x2(oacc[mbd][4 * jq + 2] * inv, oacc[mbd][4 * jq + 3] * inv)};
        *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)(
            sbase + rw * ROWB + (((4 * mbd + jq) ^ (rw & 15)) << 4) + 8 * hf) = pk;
      }
    if (qa_e >= 0) {  // all eight rows read back before the first store
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
          out + ((size_t)b * S * Hq + h) * D, 0, (int)((uint32_t)(S - 1) * q_stride + ROWB), 0x00020000);
      const int c = ln & 15;
      u32x4_t x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (ln >> 4);
        x[i] = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(
            sbase + rr * ROWB + ((c ^ (rr & 15)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = qa_e + 4 * i + (ln >> 4);
        const uint32_t off = row < n ? (uint32_t)row * q_stride + c * 16 : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(x[i], ors, (int)off, 0, kStream ? kNt : 0);
      }
    }
  };
  // Both groups store an item's output during the next item: after reading the next item's Q
  // rows into registers (phase 0) a wave stages its output in those LDS rows, and stores it row
  // by row between the score MFMAs of its first phase with MFMAs (group A: phase 0, group B:
  // phase 1). The end of an item then holds only the KV append (group A) and B's last MFMA phase.
  // With G = 1 group A stores at the end of the item instead (staged in stage T % 2, which no
  // wave reads then): keeping its output live into the next item spills registers there.
  constexpr bool kDeferA = G != 1;
  int qa_prev = 0;
  bool pending = false;

  set_lane_offsets();
  {
    DmaLane d{};
    if constexpr (!PAGED) d = dma_lane();
    issue_k(0, 2, d);  // K(0) into its own buffer, once
  }
  fetch_q(qt_of(r) * BMPOS + 32 * (w % PB));
  wait_vmcnt<0>();  // K(0) and the first item's Q rows have landed
  for (;;) {
    q0 = qt_of(r) * BMPOS;
    qa = q0 + 32 * (w % PB);
    wave_tiles = qa < n ? (p + min(qa + 31, n - 1)) / BN + 1 : 0;
    wg_tiles = (p + min(q0 + BMPOS, n) - 1) / BN + 1;
    mask_from = (p + qa) / BN;
    const int rn = next_round(r);
    has_next = rn >= 0;
    u_pf = max(wg_tiles - 1, 1);
    qa_next = has_next ? qt_of(rn) * BMPOS + 32 * (w % PB) : 0;

    set_lane_offsets();
    bar();  // phase 0; every wave is done with the previous item, its Q rows have landed
    {
      // Q^T operand: lane holds dims 16s + 8*half .. +7 of query my_q, for s = 0..7 (the
      // row's swizzle is the K rows', so the per-lane offsets are koff's; the base is kept
      // in a register the compiler may not hoist, as for K(0))
      const bool ok = qa + (fresh_lane() & 31) < n;
      uint32_t qb = qbuf - smem0;
      asm volatile("" : "+v"(qb));
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const u32x4_t t =
            *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(koff[s2] + qb);
        qop[s2] = ok ? (t ^ qsign) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if (pending && (kDeferA || w >= 4)) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the Q rows are in registers
      store_output(qbuf, -1);  // staged only: stored between the score MFMAs below
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
    m_run = -INFINITY;
    l_half = 0.f;
    even_phase_dma(0, P0{});
    if (w < 4) {
      if (wave_tiles > 0) {
        scores(PK0{}, [&](int i) {
          if (kDeferA && pending) store_rows(qbuf, qa_prev, i);
        });
      } else if (kDeferA && pending) {
        for (int i = 0; i < 8; ++i) store_rows(qbuf, qa_prev, i);
      }
      for (int t = 0; t < wg_tiles; t += 2) {
        tile_a(t, P0{});
        if (t + 1 < wg_tiles) tile_a(t + 1, P1{});
      }
      bar();
    } else {
      bar();  // phase 1
      if (wave_tiles > 0) {
        scores(PK0{}, [&](int i) {
          if (pending) store_rows(qbuf, qa_prev, i);
        });
      } else if (pending) {
        for (int i = 0; i < 8; ++i) store_rows(qbuf, qa_prev, i);
      }
      for (int t = 0; t < wg_tiles; t += 2) {
        tile_b(t, P0{});
        if (t + 1 < wg_tiles) tile_b(t + 1, P1{});
      }
    }
    // The next item's Q rows and this item's page ids have landed (requested three phases
    // earlier); the output stays in registers until the next item's phase 0 (or the end).
    wait_vmcnt<0>();
    if (!kDeferA && w < 4)
      store_output(smem0 + (uint32_t)(wg_tiles & 1) * 2 * TILE + w * 32 * ROWB, qa);
    qa_prev = qa;
    pending = true;
    if constexpr (!PAGED) {
      if (w < 4) {
        if constexpr (G == 1)
          append_rows(q0, fresh_lane() + kWave * w, 4 * kWave);
        else
          append_from_lds();
      }
    }
    if (!has_next) break;
    r = rn;
  }
  if (kDeferA || w >= 4) store_output(qbuf, qa);  // no next item: the Q rows are free
  wait_vmcnt<0>();
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

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 0;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

template <int G, bool PAGED>
static int launch_g(const void* q, const void* k, const void* v, void* out, void* k_cache,
                    void* v_cache, const int32_t* page_table, const int32_t* past_lens,
                    const int32_t* new_lens, int max_pages, int B, int S, int Hq, int Hkv,
                    float scale, hipStream_t s) {
  constexpr int BMPOS = 256 / G;
  const int n_qtiles = (S + BMPOS - 1) / BMPOS;
  const int cus = device_cus();
  if (cus <= 0) return GQA_ERR_LAUNCH;
  // One resident workgroup per compute unit: nbkv pairs x rows_per_round workgroups each
  // (at least one workgroup per pair; never more rows than q-tiles).
  const int nbkv = B * Hkv;
  const int rows = std::max(1, std::min(cus / nbkv, n_qtiles));
  hipLaunchKernelGGL((prefill_causal_kernel<G, PAGED>), dim3((unsigned)(nbkv * rows)),
                     dim3(prefill::THREADS), 0, s, (const bf16_t*)q, (const bf16_t*)k,
                     (const bf16_t*)v, (bf16_t*)out, (bf16_t*)k_cache, (bf16_t*)v_cache,
                     page_table, past_lens, new_lens, max_pages, S, Hq, Hkv, scale * kLog2e,
                     n_qtiles, nbkv, rows);
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
