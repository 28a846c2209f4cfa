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
constexpr int LOADS = 2 * TILE / (16 * THREADS);  // DMA loads per thread per tile (4)
constexpr float kLazy = 8.0f;   // log2 growth tolerated before rescaling O

// Row swizzles (16-byte chunk index XOR): K rows are read 16 at a time at one chunk,
// V rows 4 at a time over 4 chunks (transpose reads).
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }
}  // namespace prefill

template <int G>
__global__ __launch_bounds__(prefill::THREADS) void prefill_causal_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ out, int S, int Hq, int Hkv, float scale_log2, int n_qtiles) {
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
  const int qa = q0 + 32 * (w % PB);  // first query position of this wave
  const int my_q = qa + l32;          // the query this lane's softmax state belongs to

  const int wave_tiles = qa < S ? (min(qa + 31, S - 1)) / BN + 1 : 0;
  const int wg_tiles = (min(q0 + BMPOS, S) - 1) / BN + 1;

  const size_t kv_row_stride = (size_t)Hkv * D;  // elements between consecutive tokens
  const bf16_t* k_base = k + (size_t)b * S * kv_row_stride + (size_t)kvh * D;
  const bf16_t* v_base = v + (size_t)b * S * kv_row_stride + (size_t)kvh * D;

  // Q^T operand: lane holds dims 16s + 8*half .. +7 of query my_q, for s = 0..7.
  u32x4_t qop[8];
  {
    const bool ok = my_q < S;
    const bf16_t* qrow = q + (((size_t)b * S + (ok ? my_q : 0)) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4_t t = *(const u32x4_t*)(qrow + 16 * s + 8 * half);
      qop[s] = ok ? t : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  float m_run = -INFINITY;
  float l_half = 0.f;

  auto issue_tile = [&](int kt, int st) {
#pragma unroll
    for (int ii = 0; ii < LOADS; ++ii) {
      const int wi = ii * WAVES + w;   // wave instruction index: 0..15 K, 16..31 V
      const bool is_v = wi >= 16;
      const int row = 4 * (wi & 15) + (lane >> 4);
      const int chunk = (lane & 15) ^ (is_v ? v_swz(row) : k_swz(row));
      const int key = min(kt * BN + row, S - 1);
      const bf16_t* src = (is_v ? v_base : k_base) + (size_t)key * kv_row_stride + chunk * 8;
      lds_dma16(src, &smem[st][is_v ? 1 : 0][(wi & 15) * 1024]);
    }
  };

  auto compute_tile = [&](int kt, int st, bool diag) {
    const char* ks = smem[st][0];
    const char* vs = smem[st][1];
    // ---- S^T = K Q^T : two 32-key blocks ----
    f32x16_t sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = f32x16_t{};
      const int row = 32 * mb + l32;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4_t a = *(const u32x4_t*)(ks + row * ROWB + (((2 * s + half) ^ k_swz(row)) << 4));
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, qop[s]),
                                                           sacc[mb], 0, 0, 0);
      }
    }
    // ---- online softmax on this lane's query ----
    float sv[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = sacc[mb][j] * scale_log2;
        if (diag) {
          const int key = kt * BN + 32 * mb + 8 * (j >> 2) + 4 * half + (j & 3);
          x = key > my_q ? -INFINITY : x;
        }
        sv[mb][j] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new > m_run + kLazy) ? m_new : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_use;
    float psum = 0.f;
    u32x4_t pop[4];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[sp >> 1][8 * (sp & 1) + i] - m_use);
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
    // ---- O^T += V^T P^T ----
    const int g16 = lane >> 4;
    const int i16 = lane & 15;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
#pragma unroll
      for (int mbd = 0; mbd < 4; ++mbd) {
        const int chunk = 4 * mbd + 2 * (g16 & 1) + ((i16 & 3) >> 1);
        const int sub = (i16 & 1) * 8;
        const int row0 = 16 * sp + 4 * (g16 >> 1) + (i16 >> 2);
        const int row1 = row0 + 8;
        const s16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vs + row0 * ROWB + ((chunk ^ v_swz(row0)) << 4) + sub));
        const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vs + row1 * ROWB + ((chunk ^ v_swz(row1)) << 4) + sub));
        const u32x2_t a0 = __builtin_bit_cast(u32x2_t, t0);
        const u32x2_t a1 = __builtin_bit_cast(u32x2_t, t1);
        const u32x4_t a = {a0[0], a0[1], a1[0], a1[1]};
        oacc[mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                            __builtin_bit_cast(bf16x8_t, pop[sp]),
                                                            oacc[mbd], 0, 0, 0);
      }
    }
  };

  // Same stage handshake as the decode kernel: per-wave vmcnt, then a bare barrier,
  // so the next tile's DMA stays in flight while this one is used.
  issue_tile(0, 0);
  for (int kt = 0; kt < wg_tiles; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < wg_tiles) {
      issue_tile(kt + 1, st ^ 1);
      wait_vmcnt<LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (kt < wave_tiles) compute_tile(kt, st, kt == wave_tiles - 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  }

  // ---- epilogue: O = O^T / l, bf16, 4 consecutive dims per store ----
  if (wave_tiles == 0 || my_q >= S) return;
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

template <int G>
static int launch_g(const void* q, const void* k, const void* v, void* out, int B, int S, int Hq,
                    int Hkv, float scale, hipStream_t s) {
  constexpr int BMPOS = 256 / G;
  const int n_qtiles = (S + BMPOS - 1) / BMPOS;
  dim3 grid((unsigned)(B * Hkv), (unsigned)n_qtiles);
  hipLaunchKernelGGL((prefill_causal_kernel<G>), grid, dim3(prefill::THREADS), 0, s,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)out, S, Hq,
                     Hkv, scale * kLog2e, n_qtiles);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

int launch_prefill(const void* q, const void* k, const void* v, void* out, int B, int S, int Hq,
                   int Hkv, int D, float scale, hipStream_t s) {
  if (D != prefill::D) return GQA_ERR_UNSUPPORTED;
  switch (Hq / Hkv) {
    case 1: return launch_g<1>(q, k, v, out, B, S, Hq, Hkv, scale, s);
    case 2: return launch_g<2>(q, k, v, out, B, S, Hq, Hkv, scale, s);
    case 4: return launch_g<4>(q, k, v, out, B, S, Hq, Hkv, scale, s);
    case 8: return launch_g<8>(q, k, v, out, B, S, Hq, Hkv, scale, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

}  // namespace gqa
