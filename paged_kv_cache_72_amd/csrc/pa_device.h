// pa_device.h -- small device-side helpers shared by the HIP kernels of
// libpa.so: vector types, exact fp8 -> binary16 widening, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
// LDS-qualified pointers: stores through them provably leave global memory
// alone, so uniform loads of read-only tables can stay scalar loads.
typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for the running max
constexpr float kLazy = 8.0f;         // rescale only when the max grows by > 2^8

__device__ __forceinline__ half4_t halves_of(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(half4_t, make_uint2(lo, hi));
}

// 4 e4m3fn bytes -> 4 binary16 values (exact: every e4m3fn value is a binary16 value).
__device__ __forceinline__ half4_t e4m3x4_to_half4(uint32_t w) {
  const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  const float4_t f = {a.x, a.y, b.x, b.y};
  return __builtin_convertvector(f, half4_t);
}

// 4 e5m2 bytes -> 4 binary16 values: e5m2 is binary16 with the low 8 mantissa
// bits dropped, so byte b widens to the bits b << 8 (NaN and infinity included).
__device__ __forceinline__ half4_t e5m2x4_to_half4(uint32_t w) {
  const uint32_t lo = ((w << 8) & 0x0000FF00u) | ((w << 16) & 0xFF000000u);
  const uint32_t hi = ((w >> 8) & 0x0000FF00u) | (w & 0xFF000000u);
  return halves_of(lo, hi);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int clamp_len(int len, int cap) {
  return len < 0 ? 0 : (len > cap ? cap : len);
}

}  // namespace pa
