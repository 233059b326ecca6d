// Per-tensor FP8-E4M3 quantisation steps shared by the quantiser and the GEMM
// that quantises X itself ("Deploying 2:4 Sparsity with FP8 on Hopper",
// pipeline step 3 and "Troubleshooting quick hits"): the magnitude key of a
// bf16 value, the scale from the largest key, and the cast of 8 values.
#pragma once
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

}  // namespace sp24
