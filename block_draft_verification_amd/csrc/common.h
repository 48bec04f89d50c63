// Shared device helpers for the verify-pass kernels (gfx950, wave64).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
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

// two fp32 -> two fp16 (round to nearest even), packed low-first
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// two bf16 (one dword) -> two fp16; exact for |v| >= 2^-14 and |v| < 65520
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  return pack_f16x2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}

// Four fp8 e4m3 codes (one dword) -> four fp16 (two dwords), exact.
__device__ __forceinline__ u32x2_t fp8x4_to_f16x4(uint32_t codes) {
  u32x2_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, true));
  return r;
}

// Eight e2m1 codes (one dword, low nibble first) times a power-of-two scale
// -> eight fp16 (four dwords); exact while the scaled values stay fp16-normal.
__device__ __forceinline__ u32x4_t fp4x8_to_f16x8(uint32_t codes, float scale) {
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3));
  return r;
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

// D += A(16x32) * B(32x16); lane (r = lane%16, g = lane/16) supplies row r of
// A and column r of B for the 8 k of its group, and receives D[4g..4g+3][r].
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// D += A(32x16) * B(16x32); lane (c = lane%32, h = lane/32) supplies row c of A
// and column c of B for the 8 k of half h, and receives column c of D, value v
// at row 8*(v/4) + 4*h + v%4.  On gfx950 this shape issues at twice the rate of
// the 16x16x32 one.
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// D += A(32x64) * B(64x32) with OCP microscaling (v_mfma_scale_f32_32x32x64_f8f6f4).
// Lane (c, h) supplies row c of A and column c of B.  FP8 operands (format 0,
// e4m3): bytes 0-15 are k 16h..16h+15 and bytes 16-31 are k 32+16h..32+16h+15.
// FP4 operands (format 4, e2m1, only the low 4 dwords read): k 32h..32h+31,
// low nibble first.  The e8m0 scale of k block b (k 32b..32b+31) of a row or
// column is taken from lane half h = b.  Output layout as for 32x32x16.
// (Layout and scale attribution measured on gfx950 against a host product.)
template <int FMT_A>
__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t a, i32x8_t b, f32x16_t c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT_A, 0, 0, scale_a, 0, scale_b);
}

// MXFP8 quantisation of one 32-value block held 4 values per lane by 8
// consecutive lanes (lanes 8j .. 8j+7, values in order): X = floor(log2(amax))
// - 8 (e8m0 = X + 127, clamped), elements RNE to e4m3 after exact scaling by
// 2^-X, saturated at +-448.  Returns the 4 codes (byte i = value i).
__device__ __forceinline__ uint32_t mx8_quant4(f32x4_t v, uint32_t &e8) {
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  a = fmaxf(a, __shfl_xor(a, 4));
  int X = a > 0.f ? __builtin_amdgcn_frexp_expf(a) - 1 - 8 : -127;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  e8 = (uint32_t)(X + 127);
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(__builtin_ldexpf(v[i], -X), -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
}

// Workgroup barrier without __syncthreads()'s global-memory fence, which on
// gfx950 waits for every outstanding global load (vmcnt(0)) and so drains
// any prefetch in flight.  Callers wait for the loads they need themselves;
// this waits for the wave's own LDS operations, then meets the other waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
}

// Kernel arguments sit in memory that waves read with scalar loads, which the
// compiler places where each value is first used; a load whose line is not in
// the scalar cache yet costs a round trip to L2 or memory, and a kernel whose
// argument uses are spread out pays several of them in a row.  pin_args, at
// kernel entry, makes every argument dword live there, so all the loads go out
// together and later uses hit the scalar cache.
template <class T>
__device__ __forceinline__ void pin_arg(const T &v) {
  if constexpr (sizeof(T) == 4 || sizeof(T) == 8) {
    asm volatile("" ::"s"(v));
  } else {
    static_assert(sizeof(T) % 4 == 0, "dword-sized argument");
    const uint32_t *p = reinterpret_cast<const uint32_t *>(&v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(p[i]));
  }
}
template <class... T>
__device__ __forceinline__ void pin_args(const T &...v) {
  (pin_arg(v), ...);
}

__device__ __forceinline__ void set_error(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// max / sum of x over lanes l and l ^ 32 (the two halves of the wave), in
// every lane: v_permlane32_swap exchanges the halves of its two operands, so
// with x in both, the two results hold x[l] and x[l ^ 32] in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// argmax pair ordering: larger value wins, lower index on equal values.
__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return (v > bv) | ((v == bv) & (i < bi));  // bitwise: no short-circuit branches
}

// Measurement hook: while `start` is set (a context timing one kernel class,
// spec_debug_time_kernel), the next launch through launch_k records these two
// events at its own dispatch boundaries, so their difference is that kernel's
// execution time alone.  One per host thread; set and cleared by the host code
// of the C ABI around a single launch.
struct LaunchTimer {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
extern thread_local LaunchTimer g_launch_timer;

// (callers read hipGetLastError() after it, as after hipLaunchKernelGGL)
template <class K, class... A>
inline void launch_k(K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, A... args) {
  if (g_launch_timer.start && !g_launch_timer.used) {
    g_launch_timer.used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, g_launch_timer.start, g_launch_timer.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}
