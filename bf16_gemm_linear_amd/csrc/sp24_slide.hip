// SlideSparse ("SlideSparse: Fast and Flexible (2N-2):2N Structured Sparsity",
// technical summary, section 2): a (2N-2):2N weight runs on the 2:4 path.
//
// Load time: every block of 2N values along K is pruned to its 2N-2 largest
// magnitudes (ties to the lower index, as for 2:4) and laid out as N-1
// overlapping windows of 4 at stride 2 (window j covers block positions 2j ..
// 2j+3), each holding at most two of the block's values: window j takes the
// values at positions 2j, 2j+1 (no later window covers them), then fills up
// from positions 2j+2, 2j+3; what it cannot hold spills into the next window.
// The expanded weight W' (K' = K (2N-2)/N) is 2:4 along K', so the ordinary
// prune + compress keeps every value.
//
// Per call: the activations are lifted to the windows, X'[b*4(N-1) + 4j + p] =
// X[b*2N + 2j + p], inside the per-token quantiser (the page fuses the two):
// each row's scale is its own maximum over K, which lifting leaves unchanged.
#include "sp24_common.hpp"
#include "sp24_fp8.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// One thread per block of 2N values.
template <int NP>
__global__ __launch_bounds__(kThreads) void slide_prune_pack_kernel(const uint16_t* __restrict__ w,
                                                                   int64_t nblocks, uint16_t* __restrict__ out) {
  constexpr int BLK = 2 * NP, GRP = 4 * (NP - 1);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblocks; t += stride) {
    uint32_t h[BLK];
    const uint32_t* src = reinterpret_cast<const uint32_t*>(w + t * BLK);  // 4-byte aligned: BLK even
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t d = src[i];
      h[2 * i] = d & 0xFFFFu;
      h[2 * i + 1] = d >> 16;
    }
    // keep position i iff fewer than 2 values beat it (larger magnitude, or equal at a lower index)
    bool keep[BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      int beats = 0;
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        const uint32_t ai = h[i] & 0x7FFFu, aj = h[j] & 0x7FFFu;
        beats += (j != i) && (aj > ai || (aj == ai && j < i));
      }
      keep[i] = beats < BLK - 2;
    }
    // windows place the kept values whose bits are not zero (a kept +0 needs no
    // slot; -0 keeps its sign bit, as in the dense weight)
    bool nz[BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i) nz[i] = keep[i] && h[i] != 0;
    uint32_t o[GRP];
#pragma unroll
    for (int i = 0; i < GRP; ++i) o[i] = 0;
    bool taken[BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i) taken[i] = false;
#pragma unroll
    for (int j = 0; j < NP - 1; ++j) {
      int n = 0;
      // positions 2j, 2j+1: no later window covers them (the last window also takes 2j+2, 2j+3)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int pos = 2 * j + p;
        const bool must = p < 2 || j == NP - 2;
        if (must && nz[pos] && !taken[pos]) {
          o[4 * j + p] = h[pos];
          taken[pos] = true;
          ++n;
        }
      }
#pragma unroll
      for (int p = 2; p < 4; ++p) {
        const int pos = 2 * j + p;
        if (j != NP - 2 && n < 2 && nz[pos] && !taken[pos]) {
          o[4 * j + p] = h[pos];
          taken[pos] = true;
          ++n;
        }
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + t * GRP);  // GRP even
#pragma unroll
    for (int i = 0; i < GRP / 2; ++i) dst[i] = o[2 * i] | (o[2 * i + 1] << 16);
  }
}

// The 4 codes of one window (bf16 pairs d0, d1) for code type DT.
template <int DT>
__device__ __forceinline__ uint32_t qcast4(uint32_t d0, uint32_t d1, const QDiv& s) {
  const float v0 = qdiv_apply(bf16_to_f32(d0 & 0xFFFFu), s), v1 = qdiv_apply(bf16_to_f32(d0 >> 16), s);
  const float v2 = qdiv_apply(bf16_to_f32(d1 & 0xFFFFu), s), v3 = qdiv_apply(bf16_to_f32(d1 >> 16), s);
  if constexpr (DT == SP24_INT8)
    return f32_to_i8(v0) | (f32_to_i8(v1) << 8) | (f32_to_i8(v2) << 16) | (f32_to_i8(v3) << 24);
  else
    return f32x2_to_e4m3(v0, v1) | (f32x2_to_e4m3(v2, v3) << 16);
}

// Workgroup (c, b) takes the maximum over the whole of rows b, b + gridDim.y, ...
// and writes chunk c (chunk_win windows of 4 codes, one window per thread and step)
// of each row's lifted codes: a few rows are quantised by many workgroups, each
// reading its rows' maximum from L2.
template <int DT, int NP>
__global__ __launch_bounds__(kThreads) void slide_quant_rows_kernel(const uint16_t* __restrict__ x, int64_t m,
                                                                   int64_t k, uint8_t* __restrict__ q,
                                                                   float* __restrict__ scales, int64_t chunk_win) {
  constexpr int BLK = 2 * NP, GRP = 4 * (NP - 1);
  __shared__ uint32_t sh[kThreads / kWave];
  const int64_t nvec = k / 8, nwin = k / BLK * (NP - 1), kp = k / BLK * GRP;
  const int64_t w0 = (int64_t)blockIdx.x * chunk_win, w1 = min(nwin, w0 + chunk_win);
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const uint16_t* xr = x + r * k;
    const u32x4* xv = reinterpret_cast<const u32x4*>(xr);
    uint32_t mk = 0;
    int64_t i = threadIdx.x;
    for (; i + 3 * kThreads < nvec; i += 4 * kThreads) {  // four loads in flight
      const u32x4 a = xv[i], b = xv[i + kThreads], c = xv[i + 2 * kThreads], d = xv[i + 3 * kThreads];
      mk = max(mk, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
    }
    for (; i < nvec; i += kThreads) mk = max(mk, key_max8(xv[i]));
    mk = wave_max_u32(mk);
    if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = mk;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kThreads / kWave; ++j) mk = max(mk, sh[j]);
    __syncthreads();
    const QDiv s = qdiv<DT>(mk);
    if (blockIdx.x == 0 && threadIdx.x == 0) scales[r] = s.s;
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * kp);
    for (int64_t v = w0 + threadIdx.x; v < w1; v += kThreads) {
      const int64_t b = v / (NP - 1), j = v - b * (NP - 1);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(xr + b * BLK + 2 * j);  // 4-byte aligned
      qr[v] = qcast4<DT>(src[0], src[1], s);
    }
  }
}

int grid_blocks(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  if (g > 256 * 16) g = 256 * 16;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_slide_prune_pack(const uint16_t* w, int64_t n, int64_t k, int np, uint16_t* out,
                                   hipStream_t s) {
  const int64_t nblocks = n * (k / (2 * np));
  switch (np) {
#define SP24_SLIDE_PACK(NP)                                                                                 \
  case NP:                                                                                                  \
    hipLaunchKernelGGL(slide_prune_pack_kernel<NP>, dim3(grid_blocks(nblocks)), dim3(kThreads), 0, s, w,   \
                       nblocks, out);                                                                        \
    break;
    SP24_SLIDE_PACK(3) SP24_SLIDE_PACK(4) SP24_SLIDE_PACK(5) SP24_SLIDE_PACK(6) SP24_SLIDE_PACK(7)
    SP24_SLIDE_PACK(8)
#undef SP24_SLIDE_PACK
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_slide_quant_rows(int dtype, const uint16_t* x, int64_t m, int64_t k, int np, uint8_t* q,
                                   float* scales, hipStream_t s) {
  // rows over grid.y; each row's windows split over grid.x so that few rows still fill
  // about 256 workgroups (at least 256 windows each)
  const int64_t rows = m < 65535 ? m : 65535, nwin = k / (2 * np) * (np - 1);
  int64_t splits = 256 / rows;
  const int64_t most = nwin / 256;
  if (splits > most) splits = most;
  if (splits < 1) splits = 1;
  const int64_t chunk = (nwin + splits - 1) / splits;
  const dim3 blocks((unsigned)((nwin + chunk - 1) / chunk), (unsigned)rows);
  const bool i8 = dtype == SP24_INT8;
  switch (np) {
#define SP24_SLIDE_QUANT(NP)                                                                                 \
  case NP:                                                                                                   \
    if (i8)                                                                                                  \
      hipLaunchKernelGGL((slide_quant_rows_kernel<SP24_INT8, NP>), blocks, dim3(kThreads), 0, s, x, m,       \
                         k, q, scales, chunk);                                                               \
    else                                                                                                     \
      hipLaunchKernelGGL((slide_quant_rows_kernel<SP24_FP8_E4M3, NP>), blocks, dim3(kThreads), 0, s, x,       \
                         m, k, q, scales, chunk);                                                            \
    break;
    SP24_SLIDE_QUANT(3) SP24_SLIDE_QUANT(4) SP24_SLIDE_QUANT(5) SP24_SLIDE_QUANT(6) SP24_SLIDE_QUANT(7)
    SP24_SLIDE_QUANT(8)
#undef SP24_SLIDE_QUANT
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sp24
