// Bench-only ceiling kernels: a streaming HBM read and an MFMA-only loop, so that the
// attention kernels can be reported against what this GPU reaches, not only the spec.
#include "device_common.h"
#include "../../include/gqa.h"
#include "../../include/gqa_bench.h"

namespace gqa {

// NT: streaming (non-temporal) loads; otherwise ordinary loads, which allocate in every
// cache level on the way (the eviction read before a timed call).
template <int U, bool NT = true>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = src[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per workgroup
  __shared__ uint32_t red[4];
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(512) void mfma_bf16_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; it += 4) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (lane == 0) sink[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

}  // namespace gqa

extern "C" {

int gqa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks_per_cu,
                          int unroll, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks_per_cu < 1 || blocks_per_cu > 64)
    return GQA_ERR_INVALID_ARG;
  const unsigned grid = 256u * (unsigned)blocks_per_cu;
  const size_t n16 = bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  const auto* p = (const gqa::u32x4_t*)src;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(gqa::stream_read_kernel<1>, dim3(grid), dim3(256), 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(gqa::stream_read_kernel<2>, dim3(grid), dim3(256), 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(gqa::stream_read_kernel<4>, dim3(grid), dim3(256), 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(gqa::stream_read_kernel<8>, dim3(grid), dim3(256), 0, s, p, n16, sink); break;
    case 16: hipLaunchKernelGGL(gqa::stream_read_kernel<16>, dim3(grid), dim3(256), 0, s, p, n16, sink); break;
    default: return GQA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

int gqa_bench_flush_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0) return GQA_ERR_INVALID_ARG;
  hipLaunchKernelGGL((gqa::stream_read_kernel<1, false>), dim3(256u * 8u), dim3(256), 0,
                     (hipStream_t)stream, (const gqa::u32x4_t*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

int gqa_bench_mfma_bf16(float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks < 1 || iters < 4 || iters % 4 != 0) return GQA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gqa::mfma_bf16_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     sink, iters);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // extern "C"
