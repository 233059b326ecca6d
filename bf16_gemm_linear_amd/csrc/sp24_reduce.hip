// Split-K reduction: y[m, n] = bf16_rne((sum over slices z in order of
// partial[z, m, n]) * scale), scale = fp32(sx * sw) for FP8 and INT8 (sx per tensor or
// per X row, sw per tensor or per W row), 1 for BF16 and for partial sums that carry
// their group scales already.  The fixed slice order makes the result bitwise
// reproducible.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

// SPLITS > 0: the slice count is a compile-time constant and every slice's load of
// a vector is in flight before the first add (the sum is still taken in slice order);
// SPLITS == 0: any count, one slice at a time.
template <int SPLITS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, int64_t mn, int64_t n,
                                                            const float* __restrict__ x_scale,
                                                            const float* __restrict__ w_scale, int xs_step,
                                                            int ws_step, uint16_t* __restrict__ y) {
  // FP8, INT8: fp32(sx * sw), sx the scale of X row i / n and sw that of W row i % n
  // (one per tensor: step 0)
  const float s0 = x_scale != nullptr ? x_scale[0] * w_scale[0] : 1.0f;
  auto scale_of = [&](int64_t i) {
    if (x_scale == nullptr || (xs_step == 0 && ws_step == 0)) return s0;
    return x_scale[(i / n) * xs_step] * w_scale[(i % n) * ws_step];
  };
  if constexpr (SPLITS > 0) splits = SPLITS;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t nvec = (mn % 4 == 0) ? mn / 4 : 0;  // 16-byte loads need every slice aligned
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    f32x4 s;
    if constexpr (SPLITS > 0) {
      f32x4 p[SPLITS];
#pragma unroll
      for (int z = 0; z < SPLITS; ++z) p[z] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(partial + z * mn + 4 * i));
      s = p[0];
#pragma unroll
      for (int z = 1; z < SPLITS; ++z) s += p[z];
    } else {
      s = *reinterpret_cast<const f32x4*>(partial + 4 * i);
      for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(partial + z * mn + 4 * i);
    }
    u32x2 o{f32_to_bf16_rne(s[0] * scale_of(4 * i)) | (f32_to_bf16_rne(s[1] * scale_of(4 * i + 1)) << 16),
            f32_to_bf16_rne(s[2] * scale_of(4 * i + 2)) | (f32_to_bf16_rne(s[3] * scale_of(4 * i + 3)) << 16)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(y + 4 * i));
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
  // E4M3 and INT8 carry scales, unless the partial sums were scaled per group already
  const bool scaled = a.dtype != SP24_BF16 && a.group_units == 0;
  const float* xs = scaled ? a.x_scale : nullptr;
  const float* ws = scaled ? a.w_scale : nullptr;
  // the usual slice counts with every slice's load in flight at once (the decode
  // down-projection at m = 64, K in 4: 4.6 us with one slice at a time)
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((int)blocks), dim3(256), 0, s, a.partial, split_k, mn, (int64_t)a.n, xs, ws,
                       a.x_scale_step, a.w_scale_step, a.y);
  };
  switch (split_k) {
    case 2: go(splitk_reduce_kernel<2>); break;
    case 4: go(splitk_reduce_kernel<4>); break;
    case 8: go(splitk_reduce_kernel<8>); break;
    default: go(splitk_reduce_kernel<0>); break;
  }
  return hipGetLastError();
}

}  // namespace sp24
