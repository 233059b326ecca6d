// 2:4 prune + compress and decompress kernels.
//
// Pruning keeps the two largest-magnitude values of every 4 contiguous values
// along K ("Deploying 2:4 Sparsity with FP8 on Hopper", pipeline step 4 and
// Practical Example 1); ties go to the lower index.  The work is one pass over
// W: the row-major [n, k] weight (k % 32 == 0) is read and the kept values
// written as linear streams, and each metadata word goes to its place in the
// K-blocked storage order.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

// Kept positions (i0 < i1) of one group from its four magnitude keys: the
// first maximum, then the first maximum of the other three.
__device__ __forceinline__ void keep_pair(const uint32_t a[4], int& i0, int& i1) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (a[i] > a[p]) p = i;
  int q = (p == 0) ? 1 : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i != p && a[i] > a[q]) q = i;
  i0 = p < q ? p : q;
  i1 = p < q ? q : p;
}

// Thread t owns 16 bytes of W (8 values, 2 groups) and writes 8 bytes of
// kept values and one byte of nibbles; the four threads of a metadata word
// (consecutive lanes) combine their bytes with shuffles and the first writes
// the word.  Every load and value store of a wave is one contiguous 1 KB or
// 512 B piece.  nchunks = n * k / 8 is a multiple of 4, so the four threads
// of a word are always in the same wave and all active together.
__global__ __launch_bounds__(256) void prune_compress_kernel(const u32x4* __restrict__ w,
                                                             int64_t n, int64_t words,
                                                             u32x2* __restrict__ values,
                                                             uint32_t* __restrict__ meta) {
  const int64_t nchunks = n * words * 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // the stride is a multiple of 256, so every thread keeps its place in its word
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nchunks; t += stride) {
    const u32x4 in = w[t];
    uint32_t out[2];
    uint32_t nibs = 0;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t d0 = in[2 * g], d1 = in[2 * g + 1];
      const uint32_t h[4] = {d0 & 0xFFFFu, d0 >> 16, d1 & 0xFFFFu, d1 >> 16};
      const uint32_t a[4] = {h[0] & 0x7FFFu, h[1] & 0x7FFFu, h[2] & 0x7FFFu, h[3] & 0x7FFFu};
      int i0, i1;
      keep_pair(a, i0, i1);
      uint32_t v0 = h[0], v1 = h[0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i == i0) v0 = h[i];
        if (i == i1) v1 = h[i];
      }
      out[g] = v0 | (v1 << 16);
      nibs |= (uint32_t)(i0 | (i1 << 2)) << (4 * g);
    }
    values[t] = u32x2{out[0], out[1]};
    // chunk c of a word holds groups 2c, 2c+1: its byte goes to bits 8c..8c+7
    const int c = (int)(t & 3);
    uint32_t word = nibs << (8 * c);
    word |= (uint32_t)__shfl_xor((int)word, 1, 64);
    word |= (uint32_t)__shfl_xor((int)word, 2, 64);
    if (c == 0) {
      const int64_t wi = t >> 2, r = wi / words;
      meta[meta_index(r, wi - r * words, n, words)] = word;
    }
  }
}

// One thread per metadata word: 16 kept values -> 32 dense values.
template <int ESZ>
__global__ __launch_bounds__(256) void decompress_kernel(const uint8_t* __restrict__ values,
                                                         const uint32_t* __restrict__ meta,
                                                         int64_t n, int64_t words,
                                                         uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t nwords = n * words;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nwords; t += stride) {
    const int64_t r = t / words;
    const uint32_t word = meta[meta_index(r, t - r * words, n, words)];
    if constexpr (ESZ == 2) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(values + t * 32);
      u32x4 va = vp[0], vb = vp[1];
      uint32_t v[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
      uint32_t o[16];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t nib = (word >> (4 * g)) & 0xFu;
        const uint32_t i0 = nib & 3u, i1 = nib >> 2;
        uint32_t h[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i == (int)i0) h[i] = v[g] & 0xFFFFu;
          if (i == (int)i1) h[i] = v[g] >> 16;
        }
        o[2 * g] = h[0] | (h[1] << 16);
        o[2 * g + 1] = h[2] | (h[3] << 16);
      }
      u32x4* op = reinterpret_cast<u32x4*>(out + t * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) op[j] = u32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
    } else {
      const u32x4 va = *reinterpret_cast<const u32x4*>(values + t * 16);
      uint32_t o[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t pair = (va[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
        const uint32_t nib = (word >> (4 * g)) & 0xFu;
        const uint32_t i0 = nib & 3u, i1 = nib >> 2;
        uint32_t b[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i == (int)i0) b[i] = pair & 0xFFu;
          if (i == (int)i1) b[i] = pair >> 8;
        }
        o[g] = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      }
      u32x4* op = reinterpret_cast<u32x4*>(out + t * 32);
      op[0] = u32x4{o[0], o[1], o[2], o[3]};
      op[1] = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  const int64_t cap = 256 * 16;  // 16 workgroups per CU on 256 CUs; the kernels grid-stride
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

// Counts the nibbles that are not a valid kept pair (i0 < i1: 4, 8, 9, 12, 13, 14)
// and adds the count to *bad with one atomic per wave.
__global__ __launch_bounds__(256) void check_meta_kernel(const uint32_t* __restrict__ meta,
                                                         int64_t nwords, uint32_t* __restrict__ bad) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t cnt = 0;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nwords; t += stride) {
    const uint32_t word = meta[t];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t nib = (word >> (4 * g)) & 0xFu;
      cnt += (nib & 3u) >= (nib >> 2) ? 1u : 0u;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += (uint32_t)__shfl_xor((int)cnt, off, 64);
  if ((threadIdx.x & 63) == 0 && cnt != 0) atomicAdd(bad, cnt);
}

}  // namespace

hipError_t launch_prune_compress(const uint16_t* w, int64_t n, int64_t k, uint16_t* values,
                                 uint32_t* meta, hipStream_t s) {
  const int64_t nwords = n * (k / 32);
  hipLaunchKernelGGL(prune_compress_kernel, dim3(grid_for(nwords * 4, 256)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(w), n, k / 32, reinterpret_cast<u32x2*>(values),
                     meta);
  return hipGetLastError();
}

hipError_t launch_check_meta(const uint32_t* meta, int64_t n, int64_t k, uint32_t* bad,
                             hipStream_t s) {
  const int64_t nwords = n * (k / 32);
  hipLaunchKernelGGL(check_meta_kernel, dim3(grid_for(nwords, 256)), dim3(256), 0, s, meta, nwords, bad);
  return hipGetLastError();
}

hipError_t launch_decompress(int dtype, const void* values, const uint32_t* meta, int64_t n,
                             int64_t k, void* out, hipStream_t s) {
  const int64_t nwords = n * (k / 32);
  if (dtype == SP24_BF16)
    hipLaunchKernelGGL(decompress_kernel<2>, dim3(grid_for(nwords, 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(values), meta, n, k / 32,
                       static_cast<uint8_t*>(out));
  else
    hipLaunchKernelGGL(decompress_kernel<1>, dim3(grid_for(nwords, 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(values), meta, n, k / 32,
                       static_cast<uint8_t*>(out));
  return hipGetLastError();
}

}  // namespace sp24
