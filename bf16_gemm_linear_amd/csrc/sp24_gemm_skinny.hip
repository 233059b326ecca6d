// Small-m ("decode") GEMM kernels: Y[m, n] = sum_k X[m, k] W[n, k].
//
// At decode sizes the product streams the weight once and is bound by HBM
// bandwidth, so the kernel is organised around coalesced weight loads and as
// many loads in flight as possible; MFMA throughput is irrelevant here.
//
// Instruction mapping.  The sparse matrix instruction takes the compressed
// operand as "A" and the dense one as "B", so W (compressed, 16 rows) is A and
// X (16 tokens) is B; the 16x16 accumulator is a tile of Y^T:
//   lane l, accumulator register i  <->  n = 4*(l/16) + i,  m = l % 16.
// A lane of A holds row l%16 and, for lane group q = l/16, one 32-wide slice
// of K with its 8 index nibbles (one metadata word).  B lane l holds token
// l%16 and two 16-byte halves of K taken from the slices of lane groups
// q/2 and q/2 + 2 (the B layout measured on gfx950 with one-hot probes).
//
// K permutation.  Within a "chunk" of T units (a unit = 128 values of K, one
// metadata word per lane group), lane group q takes the contiguous K range
// [kb + 32*T*q, kb + 32*T*(q+1)) and unit u of the chunk reads its u-th
// 32-slice.  A and B use the same map, so the sum over K is unchanged while
// every lane reads contiguous weight bytes: 16*T compressed values and T
// metadata words per lane; activations come in 16-byte pieces.
//
// K split.  Chunks are dealt round-robin to the waves of a workgroup (and to
// grid.z slices when split_k > 1); wave partial tiles are reduced through LDS
// in a fixed wave order, split-K partials by a second kernel in a fixed slice
// order, so results are bitwise reproducible.
//
// The dense baseline (W uncompressed, dense MFMA) shares the structure.
//
// INT8 takes the integer forms of the E4M3 instructions, with the same operand
// layouts; products are summed exactly in int32 and converted to fp32 once,
// after the K loop, before the wave reduction.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

__device__ __forceinline__ i32x8 cat(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x16 as_bf16x16(i32x4 a, i32x4 b) {
  return __builtin_bit_cast(bf16x16, cat(a, b));
}

// Element offset (within a row of X) of the v-th 16-byte piece of unit u for a
// lane of group q.  Dense instructions pair A and B slots one to one, so B
// mirrors A's contiguous slice.  The sparse instructions' B operand is split
// in two halves: half h of lane group q holds instruction K
// [h*Kt/2 + q*Kt/8, +Kt/8) (Kt = 128 for fp8, 64 for bf16), which belongs to
// the A slice of lane group (q >> 1) + 2h at offset (q & 1) * Kt/8.
template <int DT, bool SPARSE, int T>
__device__ __forceinline__ int x_piece(int kb, int q, int u, int v) {
  if constexpr (SPARSE) {
    if constexpr (DT != SP24_BF16) {  // one-byte codes (E4M3 or INT8)
      return kb + 32 * T * ((q >> 1) + 2 * v) + 32 * u + 16 * (q & 1);
    } else {
      const int h = v >> 1, half = v & 1;  // instruction h of the unit, B half
      return kb + 32 * T * ((q >> 1) + 2 * half) + 32 * u + 16 * h + 8 * (q & 1);
    }
  } else {
    constexpr int ESZ = DT == SP24_BF16 ? 2 : 1;
    return kb + 32 * T * q + 32 * u + v * (16 / ESZ);
  }
}

// Registers of one chunk of T units for RB row blocks (16 rows of W each) and
// MB token blocks (16 rows of X each).
template <int DT, bool SPARSE, int T, int RB, int MB>
struct Chunk {
  static constexpr int ESZ = DT == SP24_BF16 ? 2 : 1;
  // 16-byte vectors per lane per unit: compressed W 16*ESZ bytes (dense 32*ESZ), X 32*ESZ
  static constexpr int WV = (SPARSE ? 16 : 32) * ESZ / 16;
  static constexpr int XV = 32 * ESZ / 16;
  i32x4 wv[RB][T * WV];
  uint32_t mt[RB][SPARSE ? T : 1];
  i32x4 xv[MB][T * XV];
};

// Issue every load of one chunk.  Plain (cached) loads: one load instruction
// covers only part of each 128-byte line of a weight row and the rest of the
// line arrives with the chunk's other loads, so the line must stay cached in
// between (non-temporal loads measured ~1.4x slower here).
template <int DT, bool SPARSE, int T, int RB, int MB>
__device__ __forceinline__ void load_chunk(Chunk<DT, SPARSE, T, RB, MB>& r,
                                           const uint8_t* __restrict__ w,
                                           const uint32_t* __restrict__ meta,
                                           const uint8_t* __restrict__ x, int n0, int m0, int kb,
                                           int lane, int N, int M, int K) {
  using C = Chunk<DT, SPARSE, T, RB, MB>;
  constexpr int ESZ = C::ESZ, WV = C::WV, XV = C::XV;
  const int q = lane >> 4, r16 = lane & 15;
  const int kq = kb + 32 * T * q;  // first K of this lane group's contiguous slice
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int row = n0 + rb * 16 + r16;
    row = row < N ? row : N - 1;  // ragged n: clamp the load, the store is masked
    const uint8_t* wp;
    if constexpr (SPARSE) {
      // T consecutive words from word kq / 32; T = 4 and T = 2 stay inside one
      // 128-K block (kb is a multiple of 128), T = 1 and 3 take word by word
      const int w0 = kq / 32;
      const uint32_t* mp = meta + (size_t)(w0 >> 2) * N * 4 + (size_t)row * 4 + (w0 & 3);
      if constexpr (T == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(mp);
        r.mt[rb][0] = v[0]; r.mt[rb][1] = v[1]; r.mt[rb][2] = v[2]; r.mt[rb][3] = v[3];
      } else if constexpr (T == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(mp);
        r.mt[rb][0] = v[0]; r.mt[rb][1] = v[1];
      } else {
#pragma unroll
        for (int j = 0; j < T; ++j)
          r.mt[rb][j] = meta[(size_t)((w0 + j) >> 2) * N * 4 + (size_t)row * 4 + ((w0 + j) & 3)];
      }
      wp = w + ((size_t)row * (K / 2) + kq / 2) * ESZ;
    } else {
      wp = w + ((size_t)row * K + kq) * ESZ;
    }
#pragma unroll
    for (int j = 0; j < T * WV; ++j) r.wv[rb][j] = *reinterpret_cast<const i32x4*>(wp + 16 * j);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + mb * 16 + r16;
    if (m < M) {
      const uint8_t* xr = x + (size_t)m * K * ESZ;
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int v = 0; v < XV; ++v)
          r.xv[mb][u * XV + v] =
              *reinterpret_cast<const i32x4*>(xr + x_piece<DT, SPARSE, T>(kb, q, u, v) * ESZ);
    } else {
#pragma unroll
      for (int j = 0; j < T * XV; ++j) r.xv[mb][j] = i32x4{0, 0, 0, 0};
    }
  }
}

template <int DT, bool SPARSE, int T, int RB, int MB>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[RB][MB], const Chunk<DT, SPARSE, T, RB, MB>& r) {
#pragma unroll
  for (int u = 0; u < T; ++u) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (SPARSE && DT == SP24_FP8_E4M3) {
          acc[rb][mb] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(
              r.wv[rb][u], cat(r.xv[mb][2 * u], r.xv[mb][2 * u + 1]), acc[rb][mb], (int)r.mt[rb][u], 0,
              0);
        } else if constexpr (SPARSE && DT == SP24_BF16) {
          // groups 0..3 of the word (first 16 K of the slice), then groups 4..7
          acc[rb][mb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
              as_bf16x8(r.wv[rb][2 * u]), as_bf16x16(r.xv[mb][4 * u], r.xv[mb][4 * u + 1]),
              acc[rb][mb], (int)r.mt[rb][u], 0, 0);
          acc[rb][mb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
              as_bf16x8(r.wv[rb][2 * u + 1]), as_bf16x16(r.xv[mb][4 * u + 2], r.xv[mb][4 * u + 3]),
              acc[rb][mb], (int)r.mt[rb][u], 0, 1);
        } else if constexpr (SPARSE && DT == SP24_INT8) {
          acc[rb][mb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_smfmac_i32_16x16x128_i8(
              r.wv[rb][u], cat(r.xv[mb][2 * u], r.xv[mb][2 * u + 1]),
              __builtin_bit_cast(i32x4, acc[rb][mb]), (int)r.mt[rb][u], 0, 0));
        } else if constexpr (!SPARSE && DT == SP24_INT8) {
          // dense INT8: two instructions of K=64, 16 bytes per lane group each
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[rb][mb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(
                r.wv[rb][2 * u + h], r.xv[mb][2 * u + h], __builtin_bit_cast(i32x4, acc[rb][mb]), 0, 0, 0));
        } else if constexpr (!SPARSE && DT == SP24_FP8_E4M3) {
          acc[rb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              cat(r.wv[rb][2 * u], r.wv[rb][2 * u + 1]), cat(r.xv[mb][2 * u], r.xv[mb][2 * u + 1]),
              acc[rb][mb], 0, 0, 0, 0, 0, 0);
        } else {
          // dense bf16: 4 instructions of K=32 (8 values per lane group each)
#pragma unroll
          for (int h = 0; h < 4; ++h)
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(r.wv[rb][4 * u + h]), as_bf16x8(r.xv[mb][4 * u + h]), acc[rb][mb], 0, 0, 0);
        }
      }
    }
  }
}

template <int DT, bool SPARSE, int T, int RB, int MB>
__device__ __forceinline__ void one_chunk(f32x4 (&acc)[RB][MB], const uint8_t* __restrict__ w,
                                          const uint32_t* __restrict__ meta,
                                          const uint8_t* __restrict__ x, int n0, int m0, int kb,
                                          int lane, int N, int M, int K) {
  Chunk<DT, SPARSE, T, RB, MB> r;
  load_chunk(r, w, meta, x, n0, m0, kb, lane, N, M, K);
  mma_chunk(acc, r);
}

// RB x MB tiles of 16x16 per wave; NW waves per workgroup split K; BATCH
// chunks of loads are issued before their matrix instructions.
template <int DT, bool SPARSE, int RB, int MB, int NW, int BATCH, bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
    const uint32_t* __restrict__ meta, const float* __restrict__ x_scale,
    const float* __restrict__ w_scale, uint16_t* __restrict__ y, float* __restrict__ partial,
    int M, int N, int K, int xs_step, int ws_step) {
  constexpr int TILE = RB * MB * 256;  // floats per wave tile
  __shared__ float red[NW * TILE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * (RB * 16), m0 = blockIdx.y * (MB * 16);

  f32x4 acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunks of 512 K (4 units) are dealt round-robin to the splits*NW waves
  // working on this tile; a last partial chunk of 1-3 units goes to the next
  // wave in the rotation.
  const int units = K / 128;
  const int full = units / 4, tail = units % 4;
  const int workers = gridDim.z * NW;
  const int wid = blockIdx.z * NW + wave;
  for (int c = wid; c < full; c += workers * BATCH) {
    Chunk<DT, SPARSE, 4, RB, MB> r[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (c + b * workers < full)
        load_chunk(r[b], w, meta, x, n0, m0, (c + b * workers) * 512, lane, N, M, K);
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (c + b * workers < full) mma_chunk(acc, r[b]);
  }
  if (tail != 0 && wid == full % workers) {
    const int kb = full * 512;
    if (tail == 1)
      one_chunk<DT, SPARSE, 1, RB, MB>(acc, w, meta, x, n0, m0, kb, lane, N, M, K);
    else if (tail == 2)
      one_chunk<DT, SPARSE, 2, RB, MB>(acc, w, meta, x, n0, m0, kb, lane, N, M, K);
    else
      one_chunk<DT, SPARSE, 3, RB, MB>(acc, w, meta, x, n0, m0, kb, lane, N, M, K);
  }

  if constexpr (DT == SP24_INT8)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][mb][i] = i32_bits_to_f32(acc[rb][mb][i]);

  // wave tiles -> LDS, element (rb, mb, i, lane) at ((rb*MB + mb)*4 + i)*64 + lane
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * TILE + ((rb * MB + mb) * 4 + i) * 64 + lane] = acc[rb][mb][i];
  __syncthreads();

  // Output o = ((rb*MB + mb)*16 + mi)*16 + nj: consecutive threads take
  // consecutive n of one token row; waves are summed in a fixed order.
  for (int o = threadIdx.x; o < TILE; o += NW * 64) {
    const int nj = o & 15, mi = (o >> 4) & 15, blk = o >> 8;  // blk = rb*MB + mb
    const int rb = blk / MB, mb = blk % MB;
    const int src = (blk * 4 + (nj & 3)) * 64 + (nj >> 2) * 16 + mi;
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) s += red[wv * TILE + src];
    const int n = n0 + rb * 16 + nj, m = m0 + mb * 16 + mi;
    if (n < N && m < M) {
      if constexpr (PARTIAL)
        partial[((size_t)blockIdx.z * M + m) * N + n] = s;
      else
      {
        // FP8, INT8: fp32(sx * sw) with the scales of X row m and W row n (one per
        // tensor: step 0)
        const float scale = DT != SP24_BF16 ? x_scale[(size_t)m * xs_step] * w_scale[(size_t)n * ws_step] : 1.0f;
        y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(s * scale);
      }
    }
  }
}

template <int DT, bool SPARSE, int RB, int MB, int NW, int BATCH>
hipError_t launch_cfg(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(NW * 64);
  const uint8_t* x = static_cast<const uint8_t*>(a.x);
  const uint8_t* w = static_cast<const uint8_t*>(a.w);
  if (p.split_k > 1)
    hipLaunchKernelGGL((gemm_skinny_kernel<DT, SPARSE, RB, MB, NW, BATCH, true>), grid, block, 0, s,
                       x, w, a.meta, a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, a.x_scale_step,
                       a.w_scale_step);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<DT, SPARSE, RB, MB, NW, BATCH, false>), grid, block, 0, s,
                       x, w, a.meta, a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, a.x_scale_step,
                       a.w_scale_step);
  return hipGetLastError();
}

template <int DT, bool SPARSE>
hipError_t launch_dt(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  switch (p.config) {
#define SP24_SKINNY_CASE(ID, RB, MB, NW, BATCH) \
  case ID: return launch_cfg<DT, SPARSE, RB, MB, NW, BATCH>(a, p, s);
    SP24_SKINNY_CONFIGS(SP24_SKINNY_CASE)
#undef SP24_SKINNY_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  if (a.dtype == SP24_FP8_E4M3)
    return a.sparse ? launch_dt<SP24_FP8_E4M3, true>(a, p, s) : launch_dt<SP24_FP8_E4M3, false>(a, p, s);
  if (a.dtype == SP24_INT8)
    return a.sparse ? launch_dt<SP24_INT8, true>(a, p, s) : launch_dt<SP24_INT8, false>(a, p, s);
  return a.sparse ? launch_dt<SP24_BF16, true>(a, p, s) : launch_dt<SP24_BF16, false>(a, p, s);
}

}  // namespace sp24
