// Shared device helpers for the verify-pass kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Four fp8 e4m3 codes (one dword) -> four bf16 (two dwords), exact.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t codes) {
  bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
  bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
  u32x2_t r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Eight e2m1 codes (one dword, low nibble first) times a power-of-two scale
// -> eight bf16 (four dwords), exact.
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r;
}

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ void set_error(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// argmax pair ordering: larger value wins, lower index on equal values.
__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}
