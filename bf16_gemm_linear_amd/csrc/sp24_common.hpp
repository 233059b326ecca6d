// Device-side helpers shared by the libsp24 kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));

namespace sp24 {

constexpr int kWave = 64;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// INT8 products accumulate exactly in int32; the accumulators live in float
// registers as bit patterns and become fp32 values once, after the K loop.
__device__ __forceinline__ float i32_bits_to_f32(float v) { return (float)__builtin_bit_cast(int, v); }

// Two floats -> two E4M3 codes (low byte = a), after a clamp to the format's
// range; the hardware conversion rounds to nearest even and does not saturate
// by itself, so the clamp is what keeps out-of-range values finite.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Non-temporal load: for pure streams whose every load instruction covers
// whole cache lines (the bandwidth probes).
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace sp24
