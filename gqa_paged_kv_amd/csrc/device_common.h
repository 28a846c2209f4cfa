// Device helpers shared by the libgqa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 storage is a raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

// 8-bit floating-point cache elements (raw bytes): E4M3 (bias 7, no infinities) and E5M2
// (bias 15, IEEE-style specials). gfx950 converts both natively.
struct fp8e4m3_t {
  uint8_t bits;
};
struct fp8e5m2_t {
  uint8_t bits;
};
template <typename T>
constexpr bool is_fp8() {
  return sizeof(T) == 1;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) {
  return __uint_as_float(packed & 0xffff0000u);
}
// float -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Bytes 2*hi, 2*hi+1 of a word of 8-bit floats -> two floats / one packed bf16 pair (exact:
// every E4M3 and E5M2 value is a bf16 value). The conversion is the hardware's
// (v_cvt_pk_f32_fp8 / _bf8, v_cvt_scalef32_pk_bf16_fp8 / _bf8 with scale 1).
template <typename T>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, bool hi, float& a, float& b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 v;
  if constexpr (std::is_same<T, fp8e4m3_t>::value)
    v = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  else
    v = hi ? __builtin_amdgcn_cvt_pk_f32_bf8(w, true) : __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
  a = v[0];
  b = v[1];
}
template <typename T>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  bf16x2_t v;
  if constexpr (std::is_same<T, fp8e4m3_t>::value)
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  else
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// a.x*b.x + a.y*b.y + c on packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- cross-lane reductions through DPP ------------------------------------------------
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror. A 16-lane DPP row is reduced by two quad permutes and two mirrors.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}
// x of the lane N places back in the same row (row_ror:N), N = 1 .. 15.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row rotation");
  return dpp<0x120 + N>(x);
}

// ---- across the four 16-lane rows: the row-swap instructions of gfx950 -----------------
// v_permlane16_swap exchanges rows 1 and 3 of one operand with rows 0 and 2 of the other,
// v_permlane32_swap the upper half of one with the lower half of the other. With both
// operands = x, the two results of the first hold (per lane) x and the value 16 lanes away,
// those of the second x and the value 32 lanes away: VALU operations, no LDS round trip.
__device__ __forceinline__ float rows4_sum(float x) {
  const u32x2_t a = __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                false));
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const u32x2_t b = __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                false));
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float x) {
  const u32x2_t a = __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                false));
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const u32x2_t b = __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                false));
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Over all 64 lanes; every lane gets the result.
__device__ __forceinline__ float wave_sum_f32(float x) { return rows4_sum(row16_sum(x)); }
__device__ __forceinline__ float wave_max_f32(float x) { return rows4_max(row16_max(x)); }

// ---- LDS DMA (global -> LDS without VGPRs) ---------------------------------------------
// Every lane copies 16 bytes from its own global address; lane i's bytes land at
// lds_wave_base + 16*i. lds_wave_base must be uniform across the wave.
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) leaving expcnt / lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// A value every lane of the wave holds, moved to a scalar register: the compiler then
// treats what derives from it as wave-uniform (scalar loads and branches).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long uniform(long x) {
  const unsigned long long u = (unsigned long long)x;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(u & 0xffffffffu));
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(u >> 32));
  return (long)(((unsigned long long)hi << 32) | lo);
}

}  // namespace gqa
