// Split combine and the test-only gather (gfx950).
//
// combine: merges NumSplits partials (page "解锁GQA性能潜力：从批量大小敏感性到高效优化实践",
//   section "核心参数调优：PackGQA与NumSplits的协同舞蹈") with the log-sum-exp rule:
//   out = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M), M = max_s lse_s.
// gather: bit-exact copy from the paged pool to token-major K/V,
//   token t of sequence b <-> slot t % P of page page_table[b][t / P] (page
//   "TensorRT对Grouped Query Attention的支持进展", section "动态形状与KV Cache管理";
//   page "TensorRT-LLM与TensorRT核心差异解析", section 4.2.2).
#include "device_common.h"
#include "../../include/gqa.h"

namespace gqa {

// One wave per (b, h) row; lane handles dims lane, lane+64, ...
template <typename OT, int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ ws_o,
                                                     const float* __restrict__ ws_lse,
                                                     OT* __restrict__ out, int num_splits) {
  constexpr int PER = D / kWave;
  const size_t row = blockIdx.x;
  const float* lse = ws_lse + row * num_splits;
  const float* o = ws_o + row * num_splits * D;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, lse[s]);
  float num[PER];
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  float den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < num_splits; ++s) {
      const float wgt = __builtin_amdgcn_exp2f((lse[s] - M) * kLog2e);
      den += wgt;
      for (int i = 0; i < PER; ++i) num[i] = fmaf(wgt, o[(size_t)s * D + lane + kWave * i], num[i]);
    }
  }
  for (int i = 0; i < PER; ++i) {
    const float v = den > 0.f ? num[i] / den : 0.f;
    OT* dst = out + row * D + lane + kWave * i;
    if constexpr (sizeof(OT) == 2) {
      ((uint16_t*)dst)[0] = f32_to_bf16(v);
    } else {
      *dst = v;
    }
  }
}

// Copy live tokens of (b, logical page blockIdx.x) from the pool to dst[b][t][kvh][:].
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ cache,
                                                     const int32_t* __restrict__ page_table,
                                                     const int32_t* __restrict__ lens,
                                                     char* __restrict__ dst, int Hkv,
                                                     int row_bytes, int P, int max_pages) {
  const int lp = blockIdx.x;
  const int b = blockIdx.y;
  int T = lens[b];
  T = T < 0 ? 0 : (T > max_pages * P ? max_pages * P : T);
  if (lp * P >= T) return;
  const int phys = page_table[(size_t)b * max_pages + lp];
  const int chunks_row = row_bytes / 16;
  const int chunks = Hkv * P * chunks_row;
  for (int idx = threadIdx.x; idx < chunks; idx += blockDim.x) {
    const int kvh = idx / (P * chunks_row);
    const int rem = idx % (P * chunks_row);
    const int slot = rem / chunks_row;
    const int c = rem % chunks_row;
    const int t = lp * P + slot;
    if (t >= T) continue;
    const u32x4_t v = *(const u32x4_t*)(cache + (((size_t)phys * Hkv + kvh) * P + slot) * row_bytes + c * 16);
    *(u32x4_t*)(dst + (((size_t)b * max_pages * P + t) * Hkv + kvh) * row_bytes + c * 16) = v;
  }
}

int launch_combine(const float* ws_o, const float* ws_lse, void* out, int B, int Hq, int D,
                   int ns, int dtype, hipStream_t s) {
  dim3 grid((unsigned)B * Hq);
  if (dtype == GQA_BF16) {
    if (D == 128) hipLaunchKernelGGL((combine_kernel<bf16_t, 128>), grid, dim3(64), 0, s, ws_o, ws_lse, (bf16_t*)out, ns);
    else hipLaunchKernelGGL((combine_kernel<bf16_t, 64>), grid, dim3(64), 0, s, ws_o, ws_lse, (bf16_t*)out, ns);
  } else {
    if (D == 128) hipLaunchKernelGGL((combine_kernel<float, 128>), grid, dim3(64), 0, s, ws_o, ws_lse, (float*)out, ns);
    else hipLaunchKernelGGL((combine_kernel<float, 64>), grid, dim3(64), 0, s, ws_o, ws_lse, (float*)out, ns);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

int launch_gather(const void* cache, const int32_t* pt, const int32_t* lens, void* dst, int B,
                  int Hkv, int D, int P, int max_pages, int dtype, hipStream_t s) {
  const int row_bytes = D * (dtype == GQA_BF16 ? 2 : 4);
  hipLaunchKernelGGL(gather_kernel, dim3(max_pages, B), dim3(256), 0, s, (const char*)cache, pt,
                     lens, (char*)dst, Hkv, row_bytes, P, max_pages);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}


}  // namespace gqa
