/*
 * gqa_bench.h -- bench-only kernels of libgqa that measure what this GPU can
 * actually reach, reported next to the spec peaks (not part of the attention API).
 *
 * Conventions as in gqa.h: device pointers owned by the caller, work enqueued on
 * `stream`, the return value reports validation and launch only.
 */
#ifndef GQA_BENCH_H
#define GQA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes (a multiple of 16) at `src` with 128-bit loads,
 * `blocks_per_cu` x 256-thread workgroups per CU (the grid is 256 * blocks_per_cu
 * workgroups), `unroll` independent loads in flight per thread (1..16). `sink`
 * receives one 32-bit word per workgroup (an XOR of what it read) so the loads
 * cannot be elided. Achieved read bandwidth = bytes / kernel time.
 */
int gqa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks_per_cu,
                          int unroll, void* stream);

/*
 * Cache eviction before a timed call: reads `bytes` bytes (a multiple of 16) at `src` with
 * ordinary 128-bit loads, which allocate in the L2 caches and the Infinity Cache (the
 * streaming loads of gqa_bench_stream_read may bypass the latter), 8 x 256-thread
 * workgroups per CU. Pass a buffer several times the Infinity Cache (256 MB); `sink` as in
 * gqa_bench_stream_read.
 */
int gqa_bench_flush_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Back-to-back v_mfma_f32_32x32x16_bf16 on register operands: `iters` MFMAs per wave,
 * 8 waves per workgroup, `blocks` workgroups; `sink` gets one float per wave.
 * Flops = blocks * 8 * iters * 32768.
 */
int gqa_bench_mfma_bf16(float* sink, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_BENCH_H */
