// Split-K reduction: y[m, n] = bf16_rne((sum over slices z in order of
// partial[z, m, n]) * scale), scale = fp32(sx * sw) for FP8 and INT8 (sx per tensor or
// per X row).  The fixed slice order makes the result bitwise
// reproducible.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, int64_t mn, int64_t n,
                                                            const float* __restrict__ x_scale,
                                                            const float* __restrict__ w_scale, int xs_step,
                                                            uint16_t* __restrict__ y) {
  // FP8, INT8: fp32(sx * sw), sx the scale of X row i / n (one per tensor: xs_step = 0)
  const float s0 = x_scale != nullptr ? x_scale[0] * w_scale[0] : 1.0f;
  auto scale_of = [&](int64_t i) { return xs_step == 0 ? s0 : x_scale[i / n] * w_scale[0]; };
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t nvec = (mn % 4 == 0) ? mn / 4 : 0;  // 16-byte loads need every slice aligned
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    f32x4 s = *reinterpret_cast<const f32x4*>(partial + 4 * i);
    for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(partial + z * mn + 4 * i);
    u32x2 o{f32_to_bf16_rne(s[0] * scale_of(4 * i)) | (f32_to_bf16_rne(s[1] * scale_of(4 * i + 1)) << 16),
            f32_to_bf16_rne(s[2] * scale_of(4 * i + 2)) | (f32_to_bf16_rne(s[3] * scale_of(4 * i + 3)) << 16)};
    *reinterpret_cast<u32x2*>(y + 4 * i) = o;
  }
  for (int64_t i = nvec * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
    float s = partial[i];
    for (int z = 1; z < splits; ++z) s += partial[z * mn + i];
    y[i] = (uint16_t)f32_to_bf16_rne(s * scale_of(i));
  }
}

}  // namespace

hipError_t launch_splitk_reduce(const GemmArgs& a, int split_k, hipStream_t s) {
  const int64_t mn = (int64_t)a.m * a.n;
  int64_t blocks = (mn / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  const bool scaled = a.dtype != SP24_BF16;  // E4M3 and INT8 carry scales
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((int)blocks), dim3(256), 0, s, a.partial, split_k, mn,
                     (int64_t)a.n, scaled ? a.x_scale : nullptr, scaled ? a.w_scale : nullptr, a.x_scale_step,
                     a.y);
  return hipGetLastError();
}

}  // namespace sp24
