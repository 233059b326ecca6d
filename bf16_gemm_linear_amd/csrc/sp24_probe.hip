// Layout, issue-rate and bandwidth probes (see include/sp24_probe.h).
//
// The layout probe runs one matrix instruction per wave on operands read from
// memory and writes back the accumulator registers, so the host can map
// lanes, registers and sparse index bits to matrix coordinates with one-hot
// inputs.  Every access is at a fixed per-lane stride inside buffers whose
// size the caller derives from n_exp.
#include <type_traits>

#include "../../include/sp24_probe.h"
#include "sp24_common.hpp"
#include "sp24_dma.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

template <int V>
__global__ __launch_bounds__(64) void layout_kernel(const uint8_t* __restrict__ a,
                                                    const uint8_t* __restrict__ b,
                                                    const uint32_t* __restrict__ idx,
                                                    float* __restrict__ c) {
  const int64_t slot = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const i32x4 a0 = *reinterpret_cast<const i32x4*>(a + slot * 32);
  const i32x4 a1 = *reinterpret_cast<const i32x4*>(a + slot * 32 + 16);
  const i32x4 b0 = *reinterpret_cast<const i32x4*>(b + slot * 32);
  const i32x4 b1 = *reinterpret_cast<const i32x4*>(b + slot * 32 + 16);
  const int ix = (int)idx[slot];
  const i32x8 bb{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  float* out = c + slot * 16;
  if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_I8 || V == SP24_PROBE_MFMA_16x16x64_I8) {
    i32x4 acc{0, 0, 0, 0};
    if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_I8)
      acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a0, bb, acc, ix, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (float)acc[i];
  } else if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_I8 || V == SP24_PROBE_MFMA_32x32x32_I8) {
    i32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
    if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_I8)
      acc = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a0, bb, acc, ix, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = (float)acc[i];
  } else if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_FP8 || V == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID0 ||
                V == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID1 || V == SP24_PROBE_MFMA_16x16x128_FP8 ||
                V == SP24_PROBE_MFMA_16x16x32_BF16) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
    if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_FP8)
      acc = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a0, bb, acc, ix, 0, 0);
    else if constexpr (V == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID0)
      acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a0),
                                                      __builtin_bit_cast(bf16x16, bb), acc, ix, 0, 0);
    else if constexpr (V == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID1)
      acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a0),
                                                      __builtin_bit_cast(bf16x16, bb), acc, ix, 0, 1);
    else if constexpr (V == SP24_PROBE_MFMA_16x16x128_FP8) {
      const i32x8 aa{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa, bb, acc, 0, 0, 0, 0, 0, 0);
    } else
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                    __builtin_bit_cast(bf16x8, b0), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = acc[i];
  } else {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_FP8)
      acc = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a0, bb, acc, ix, 0, 0);
    else if constexpr (V == SP24_PROBE_SMFMAC_32x32x32_BF16_ABID0)
      acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                      __builtin_bit_cast(bf16x16, bb), acc, ix, 0, 0);
    else
      acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                      __builtin_bit_cast(bf16x16, bb), acc, ix, 0, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = acc[i];
  }
}

// Back-to-back instructions on register operands, four independent chains.
template <int V>
__global__ void rate_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  i32x8 b = {lane, 1, 2, 3, 4, 5, 6, lane};
  const int ix = 0x88888888 ^ lane;  // any valid-looking index pattern
  float r = 0.f;
  if constexpr (V >= SP24_PROBE_SMFMAC_16x16x128_I8) {
    constexpr bool WIDE = V == SP24_PROBE_SMFMAC_32x32x64_I8 || V == SP24_PROBE_MFMA_32x32x32_I8;
    using Acc = typename std::conditional<WIDE, i32x16, i32x4>::type;
    Acc c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_I8) {
        c0 = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c3, ix, 0, 0);
      } else if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_I8) {
        c0 = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c3, ix, 0, 0);
      } else if constexpr (V == SP24_PROBE_MFMA_16x16x64_I8) {
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a + 1, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a + 1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a + 1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a + 1, c3, 0, 0, 0);
      } else {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a + 1, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a + 1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a + 1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a + 1, c3, 0, 0, 0);
      }
    }
    for (int i = 0; i < (WIDE ? 16 : 4); ++i) r += (float)(c0[i] + c1[i] + c2[i] + c3[i]);
  } else if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_FP8 || V == SP24_PROBE_SMFMAC_32x32x32_BF16_ABID0) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      if constexpr (V == SP24_PROBE_SMFMAC_32x32x64_FP8) {
        c0 = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c3, ix, 0, 0);
      } else {
        const bf16x8 aa = __builtin_bit_cast(bf16x8, a);
        const bf16x16 bb = __builtin_bit_cast(bf16x16, b);
        c0 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(aa, bb, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(aa, bb, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(aa, bb, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(aa, bb, c3, ix, 0, 0);
      }
    }
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const i32x8 a8 = {lane, 1, 2, 3, 4, 5, 6, 7};
    for (int it = 0; it < iters; ++it) {
      if constexpr (V == SP24_PROBE_SMFMAC_16x16x128_FP8) {
        c0 = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c3, ix, 0, 0);
      } else if constexpr (V == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID0) {
        const bf16x8 aa = __builtin_bit_cast(bf16x8, a);
        const bf16x16 bb = __builtin_bit_cast(bf16x16, b);
        c0 = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(aa, bb, c0, ix, 0, 0);
        c1 = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(aa, bb, c1, ix, 0, 0);
        c2 = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(aa, bb, c2, ix, 0, 0);
        c3 = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(aa, bb, c3, ix, 0, 0);
      } else if constexpr (V == SP24_PROBE_MFMA_16x16x128_FP8) {
        c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c3, 0, 0, 0, 0, 0, 0);
      } else {
        const bf16x8 aa = __builtin_bit_cast(bf16x8, a);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, a + 1);
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, c3, 0, 0, 0);
      }
    }
    for (int i = 0; i < 4; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride)
    dst[i] = ld_nt(src + i);
}

constexpr int kReadBlocks = 256 * 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t nvec,
                                                   uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = ld_nt(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t sh[4];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

// The load path of the LDS-ring GEMM kernels without their arithmetic: a ring of
// S LDS buffers; per step a workgroup of 8 waves loads WKB KB of W (its own
// region, read once) and XKB KB of X (a region per XCD, re-read, so L2-resident)
// with global_load_lds, 16 bytes a lane, W first.  Each wave waits for its loads
// of step ks, then (BAR) the workgroup synchronises, and the loads of step
// ks + S - 1 go out, as in the GEMM kernels' rings.
constexpr int kRingWaves = 8;

template <int WKB, int XKB, int S, bool BAR>
__global__ __launch_bounds__(kRingWaves * 64) void ring_kernel(const uint8_t* __restrict__ w, int64_t w_stride,
                                                                const uint8_t* __restrict__ x, int64_t x_region,
                                                                int steps, uint32_t* __restrict__ out) {
  constexpr int PER = (WKB + XKB) / kRingWaves;
  static_assert((WKB + XKB) % kRingWaves == 0 && PER >= 1, "whole loads per wave");
  static_assert(PER * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * (WKB + XKB) * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint8_t* wp = w + (int64_t)blockIdx.x * w_stride + lane * 16;
  const uint8_t* xp = x + (int64_t)(blockIdx.x % 8) * x_region + lane * 16;
  auto issue = [&](int ks) {
    uint8_t* buf = lds + (ks % S) * (WKB + XKB) * 1024;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int g = j * kRingWaves + wave;  // load g of the step
      if (g < WKB) dma16(wp + ((int64_t)ks * WKB + g) * 1024, buf + g * 1024);
      else dma16(xp + ((((int64_t)ks * XKB + (g - WKB)) * 1024) & (x_region - 1)), buf + g * 1024);
    }
  };
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < steps) issue(p);
  uint32_t acc = 0;
  for (int ks = 0; ks < steps; ++ks) {
    const int left = steps - 1 - ks;
    wait_later<PER, S - 2>(left < S - 2 ? left : S - 2);
    if constexpr (BAR) __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ks + S - 1 < steps) issue(ks + S - 1);
    acc ^= *reinterpret_cast<const uint32_t*>(lds + (ks % S) * (WKB + XKB) * 1024 + wave * 1024 + lane * 16);
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

}  // namespace
}  // namespace sp24

using namespace sp24;

extern "C" {

int sp24_probe_mfma_layout(int variant, const void* a, const void* b, const uint32_t* idx, float* c,
                           int n_exp, void* stream) {
  if (variant < 0 || variant >= SP24_PROBE_N_VARIANTS) return SP24_ERR_MODE;
  if (!a || !b || !idx || !c) return SP24_ERR_NULL;
  if (n_exp < 1 || n_exp > (1 << 20)) return SP24_ERR_SHAPE;
  if ((((uintptr_t)a | (uintptr_t)b | (uintptr_t)idx | (uintptr_t)c) & 15u) != 0) return SP24_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* pa = static_cast<const uint8_t*>(a);
  const uint8_t* pb = static_cast<const uint8_t*>(b);
  switch (variant) {
#define SP24_LAYOUT_CASE(V) \
  case V: hipLaunchKernelGGL(layout_kernel<V>, dim3(n_exp), dim3(64), 0, s, pa, pb, idx, c); break;
    SP24_LAYOUT_CASE(0) SP24_LAYOUT_CASE(1) SP24_LAYOUT_CASE(2) SP24_LAYOUT_CASE(3)
    SP24_LAYOUT_CASE(4) SP24_LAYOUT_CASE(5) SP24_LAYOUT_CASE(6) SP24_LAYOUT_CASE(7)
    SP24_LAYOUT_CASE(8) SP24_LAYOUT_CASE(9) SP24_LAYOUT_CASE(10) SP24_LAYOUT_CASE(11)
#undef SP24_LAYOUT_CASE
  }
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_HIP;
}

int sp24_probe_mfma_rate(int variant, int iters, int blocks, int waves, float* out, void* stream) {
  if (variant < 0 || variant >= SP24_PROBE_N_VARIANTS || variant == SP24_PROBE_SMFMAC_16x16x64_BF16_ABID1 ||
      variant == SP24_PROBE_SMFMAC_32x32x32_BF16_ABID1)
    return SP24_ERR_MODE;
  if (!out) return SP24_ERR_NULL;
  if (iters < 1 || blocks < 1 || waves < 1 || waves > 16 || blocks > (1 << 20)) return SP24_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 g(blocks), blk(waves * 64);
  switch (variant) {
    case 0: hipLaunchKernelGGL(rate_kernel<0>, g, blk, 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(rate_kernel<1>, g, blk, 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL(rate_kernel<3>, g, blk, 0, s, iters, out); break;
    case 4: hipLaunchKernelGGL(rate_kernel<4>, g, blk, 0, s, iters, out); break;
    case 6: hipLaunchKernelGGL(rate_kernel<6>, g, blk, 0, s, iters, out); break;
    case 7: hipLaunchKernelGGL(rate_kernel<7>, g, blk, 0, s, iters, out); break;
    case 8: hipLaunchKernelGGL(rate_kernel<8>, g, blk, 0, s, iters, out); break;
    case 9: hipLaunchKernelGGL(rate_kernel<9>, g, blk, 0, s, iters, out); break;
    case 10: hipLaunchKernelGGL(rate_kernel<10>, g, blk, 0, s, iters, out); break;
    case 11: hipLaunchKernelGGL(rate_kernel<11>, g, blk, 0, s, iters, out); break;
  }
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_HIP;
}

int sp24_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return SP24_ERR_NULL;
  if (bytes == 0 || bytes % 16) return SP24_ERR_SHAPE;
  if ((((uintptr_t)src | (uintptr_t)dst) & 15u) != 0) return SP24_ERR_ALIGN;
  const uintptr_t a0 = (uintptr_t)src, b0 = (uintptr_t)dst;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return SP24_ERR_ALIAS;
  const int64_t nvec = (int64_t)(bytes / 16);
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(copy_kernel, dim3((int)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_HIP;
}

int sp24_probe_read_blocks(void) { return kReadBlocks; }

int sp24_probe_ring(int w_kb, int x_kb, int stages, int barrier, const void* w, size_t w_stride, const void* x,
                    size_t x_bytes, int blocks, int steps, uint32_t* out, void* stream) {
  if (!out || (w_kb > 0 && !w) || (x_kb > 0 && !x)) return SP24_ERR_NULL;
  if (blocks < 1 || blocks > 65536 || steps < 1) return SP24_ERR_SHAPE;
  if (w_kb > 0 && w_stride < (size_t)steps * w_kb * 1024) return SP24_ERR_SHAPE;
  const size_t x_region = x_bytes / 8;  // one region per XCD: a power of two of at least one step
  if (x_kb > 0 && (x_bytes % 8 != 0 || x_region < (size_t)x_kb * 1024 || (x_region & (x_region - 1)) != 0))
    return SP24_ERR_SHAPE;
  if ((((uintptr_t)w | (uintptr_t)x | (uintptr_t)out | w_stride) & 15u) != 0) return SP24_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* pw = static_cast<const uint8_t*>(w);
  const uint8_t* px = static_cast<const uint8_t*>(x);
  const dim3 g(blocks), blk(kRingWaves * 64);
  const int64_t ws = (int64_t)w_stride, xr = (int64_t)(x_region > 0 ? x_region : 1024);
#define SP24_RING_CASE(WKB, XKB, S, BAR)                                                                  \
  if (w_kb == WKB && x_kb == XKB && stages == S && (barrier != 0) == BAR) {                              \
    hipLaunchKernelGGL((ring_kernel<WKB, XKB, S, BAR>), g, blk, 0, s, pw, ws, px, xr, steps, out);        \
    return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_HIP;                                      \
  }
  SP24_PROBE_RING_SHAPES(SP24_RING_CASE)
#undef SP24_RING_CASE
  return SP24_ERR_MODE;
}

int sp24_probe_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (!src || !out) return SP24_ERR_NULL;
  if (bytes == 0 || bytes % 16) return SP24_ERR_SHAPE;
  if ((((uintptr_t)src | (uintptr_t)out) & 15u) != 0) return SP24_ERR_ALIGN;
  hipLaunchKernelGGL(read_kernel, dim3(kReadBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? SP24_OK : SP24_ERR_HIP;
}

}  // extern "C"
