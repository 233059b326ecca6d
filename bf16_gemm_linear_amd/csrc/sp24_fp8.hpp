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

// The divisor of a cast: s, and for a scale taken from the data's own largest
// magnitude (dynamic scaling) its reciprocal r = fp32(1 / s).  With fast set the
// quotient v / s is formed as q0 = v r, then one correction with the exact
// residual, q = q0 + fma(-q0, s, v) r (its sign taken from v, so that -0 stays
// -0); otherwise by IEEE float32 division.  For s = fp32(amax / 448) or
// fp32(amax / 127) with amax a finite bf16 of at least 2^-63 (key >= 0x2000) and
// every bf16 v with |v| <= amax, the corrected quotient gives the same E4M3 and
// INT8 code as the correctly rounded one (checked exhaustively over all such
// pairs on the CPU); below that amax, for infinite or NaN amax and for scales a
// caller supplies, the division is used.
struct QDiv {
  float s, r;
  bool fast;
};

__device__ __forceinline__ QDiv qdiv_static(float s) { return QDiv{s, 0.0f, false}; }

__device__ __forceinline__ QDiv qdiv_dynamic(uint32_t key, float s) {
  const bool fast = key >= 0x2000u && key < 0x7F80u;
  return QDiv{s, fast ? 1.0f / s : 0.0f, fast};
}

// From a scale and the reciprocal qdiv_dynamic gave it (0 when it took the division).
__device__ __forceinline__ QDiv qdiv_from(float s, float r) { return QDiv{s, r, r != 0.0f}; }

__device__ __forceinline__ float qdiv_apply(float v, const QDiv& q) {
  if (!q.fast) return v / q.s;
  const float q0 = v * q.r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, q.s, v), q.r, q0), v);
}

// 8 bf16 -> 8 E4M3 codes of v / s (clamped to +-448, round to nearest even).
__device__ __forceinline__ u32x2 cast8(u32x4 d, float s) {
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = f32x2_to_e4m3(bf16_to_f32(d[j] & 0xFFFFu) / s, bf16_to_f32(d[j] >> 16) / s);
  return u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
}

// The same with the divisor of a QDiv (uniform branch: both routes are written out).
__device__ __forceinline__ u32x2 cast8(u32x4 d, const QDiv& q) {
  if (!q.fast) return cast8(d, q.s);
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = f32x2_to_e4m3(qdiv_apply(bf16_to_f32(d[j] & 0xFFFFu), q), qdiv_apply(bf16_to_f32(d[j] >> 16), q));
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

__device__ __forceinline__ u32x2 cast8_i8(u32x4 d, const QDiv& q) {
  if (!q.fast) return cast8_i8(d, q.s);
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = f32_to_i8(qdiv_apply(bf16_to_f32(d[j] & 0xFFFFu), q)) |
           (f32_to_i8(qdiv_apply(bf16_to_f32(d[j] >> 16), q)) << 8);
  return u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
}

// The steps of code type DT (SP24_FP8_E4M3 or SP24_INT8).
template <int DT>
__device__ __forceinline__ float qscale(uint32_t key) {
  if constexpr (DT == SP24_INT8) return scale_from_key_i8(key);
  else return scale_from_key(key);
}

// The divisor of the scale from largest key `key` (dynamic scaling).
template <int DT>
__device__ __forceinline__ QDiv qdiv(uint32_t key) {
  return qdiv_dynamic(key, qscale<DT>(key));
}

template <int DT>
__device__ __forceinline__ u32x2 qcast8(u32x4 d, const QDiv& q) {
  if constexpr (DT == SP24_INT8) return cast8_i8(d, q);
  else return cast8(d, q);
}

template <int DT>
__device__ __forceinline__ uint8_t qcast1(uint32_t h, const QDiv& q) {
  const float v = qdiv_apply(bf16_to_f32(h), q);
  if constexpr (DT == SP24_INT8) return (uint8_t)f32_to_i8(v);
  else return (uint8_t)(f32x2_to_e4m3(v, 0.0f) & 0xFFu);
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
