// Per-tensor FP8-E4M3 quantisation steps shared by the quantiser and the GEMM
// that quantises X itself ("Deploying 2:4 Sparsity with FP8 on Hopper",
// pipeline step 3 and "Troubleshooting quick hits"): the magnitude key of a
// bf16 value, the scale from the largest key, and the cast of 8 values; and
// their symmetric INT8 counterparts (the same page's INT8 W8A8 recipe).
#pragma once
#include "sp24.h"
#include "sp24_common.hpp"

namespace sp24 {

// Largest magnitude key (bits & 0x7FFF: orders finite bf16 magnitudes exactly)
// of 8 bf16 values.
__device__ __forceinline__ uint32_t key_max8(u32x4 d) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = max(m, d[j] & 0x7FFFu);
    m = max(m, (d[j] >> 16) & 0x7FFFu);
  }
  return m;
}

// s = fp32(amax / 448), 1 when amax is 0; the division is IEEE float32.
__device__ __forceinline__ float scale_from_key(uint32_t key) {
  return key == 0 ? 1.0f : bf16_to_f32(key) / 448.0f;
}

// 8 bf16 -> 8 E4M3 codes of v / s (clamped to +-448, round to nearest even).
__device__ __forceinline__ u32x2 cast8(u32x4 d, float s) {
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = f32x2_to_e4m3(bf16_to_f32(d[j] & 0xFFFFu) / s, bf16_to_f32(d[j] >> 16) / s);
  return u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
}

// INT8: s = fp32(amax / 127), 1 when amax is 0 (IEEE float32 division).
__device__ __forceinline__ float scale_from_key_i8(uint32_t key) {
  return key == 0 ? 1.0f : bf16_to_f32(key) / 127.0f;
}

// One INT8 code: round to nearest even, then clamp to +-127 (never -128).
__device__ __forceinline__ uint32_t f32_to_i8(float v) {
  const float r = fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
  return (uint32_t)(int)r & 0xFFu;
}

// 8 bf16 -> 8 INT8 codes of v / s.
__device__ __forceinline__ u32x2 cast8_i8(u32x4 d, float s) {
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = f32_to_i8(bf16_to_f32(d[j] & 0xFFFFu) / s) | (f32_to_i8(bf16_to_f32(d[j] >> 16) / s) << 8);
  return u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
}

// The steps of code type DT (SP24_FP8_E4M3 or SP24_INT8).
template <int DT>
__device__ __forceinline__ float qscale(uint32_t key) {
  if constexpr (DT == SP24_INT8) return scale_from_key_i8(key);
  else return scale_from_key(key);
}

template <int DT>
__device__ __forceinline__ u32x2 qcast8(u32x4 d, float s) {
  if constexpr (DT == SP24_INT8) return cast8_i8(d, s);
  else return cast8(d, s);
}

template <int DT>
__device__ __forceinline__ uint8_t qcast1(uint32_t h, float s) {
  if constexpr (DT == SP24_INT8) return (uint8_t)f32_to_i8(bf16_to_f32(h) / s);
  else return (uint8_t)(f32x2_to_e4m3(bf16_to_f32(h) / s, 0.0f) & 0xFFu);
}

}  // namespace sp24
