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

typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

// 4 e4m3fn bytes -> 4 binary16 values (exact: every e4m3fn value is a binary16
// value), two at a time by gfx950's scaled packed conversion with scale 1.
// Checked against the exact widening for all 256 bytes on the device.
__device__ __forceinline__ half4_t e4m3x4_to_half4(uint32_t w) {
  const half2v_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const half2v_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return half4_t{a.x, a.y, b.x, b.y};
}

// 4 e5m2 bytes -> 4 binary16 values: e5m2 is binary16 with the low 8 mantissa
// bits dropped, so byte b widens to the bits b << 8 (infinities included; the
// conversion below gives exactly those bits for every byte that is not NaN).
__device__ __forceinline__ half4_t e5m2x4_to_half4(uint32_t w) {
  const half2v_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false);
  const half2v_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true);
  return half4_t{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int clamp_len(int len, int cap) {
  return len < 0 ? 0 : (len > cap ? cap : len);
}

}  // namespace pa
