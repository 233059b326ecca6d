// Large-m ("prefill") GEMM kernels: Y[m, n] = sum_k X[m, k] W[n, k] with
// 256 x 256 output tiles per workgroup, staged through LDS.
//
// At prefill sizes the product is bound by matrix-core throughput.  Each
// workgroup (4 waves, one per SIMD) owns a 256 (n) x 256 (m) tile of Y and
// walks K in steps of KS = 128 (fp8) or 64 (bf16) values.  A step brings, for
// every W row, 64 bytes of compressed values plus KS/32 metadata words, and
// for every X row 128 bytes; two LDS buffers alternate so the global loads of
// step k+1 are in flight while step k is multiplied.  Each wave computes a
// 128 x 128 sub-tile as 4 x 4 instructions of 32 x 32 (sparse:
// v_smfmac_f32_32x32x64_fp8_fp8 / v_smfmac_f32_32x32x32_bf16; dense baseline:
// v_mfma_f32_32x32x64_f8f6f4 / v_mfma_f32_32x32x16_bf16).
//
// Operand layouts of the 32x32 sparse instructions (measured on gfx950 with
// one-hot probes): A lane l holds W row l%32 and, for lane group q = l/32,
// the contiguous instruction-K half [q*Kt/2, (q+1)*Kt/2) with its index bits;
// B lane l holds X row l%32 and two runs of Kt/4 values, run h covering
// instruction K [h*Kt/2 + q*Kt/4, ...).  Instruction K is mapped to the
// step's K so that every fragment is one 16-byte LDS read and the index bits
// of a lane are one metadata word (fp8) or one 16-bit half of one, selected
// by abid (bf16).
//
// LDS rows are XOR-swizzled in 16-byte units so that the fragment reads of 16
// consecutive lanes hit 16 distinct bank groups.  Workgroups are mapped to
// tiles XCD by XCD and, inside an XCD, in groups of 8 tile columns, so that
// workgroups resident at the same time share W and X tiles in their XCD's L2.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int BN = 256, BM = 256, NT = 256;  // tile rows of W, rows of X, threads
constexpr int GROUP_N = 8;                   // tile columns per group in the tile order

template <int DT, bool SPARSE>
struct TiledLayout {
  static constexpr int ESZ = DT == SP24_BF16 ? 2 : 1;
  static constexpr int KS = DT == SP24_BF16 ? 64 : 128;  // K values per step
  static constexpr int WB = SPARSE ? 64 : 128;           // W bytes per row per step
  static constexpr int MWORDS = SPARSE ? KS / 32 : 0;    // metadata words per row per step
  static constexpr int XB = 128;                         // X bytes per row per step
  static constexpr int W_OFF = 0;
  static constexpr int M_OFF = W_OFF + BN * WB;
  static constexpr int X_OFF = M_OFF + BN * MWORDS * 4;
  static constexpr int STAGE = X_OFF + BM * XB;          // bytes per LDS buffer
};

// 16-byte column swizzles (see the file comment).
__device__ __forceinline__ int swz_w(int row, int c, int pieces) {
  return pieces == 4 ? (c ^ ((row >> 2) & 3)) : (c ^ ((row >> 1) & 7));
}
__device__ __forceinline__ int swz_x(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int DT, bool SPARSE>
struct StageRegs {
  using L = TiledLayout<DT, SPARSE>;
  static constexpr int WP = BN * L::WB / 16 / NT;  // 16-byte pieces of W per thread
  static constexpr int XP = BM * L::XB / 16 / NT;  // 16-byte pieces of X per thread
  i32x4 w[WP];
  i32x4 x[XP];
  uint32_t meta[SPARSE ? L::MWORDS : 1];
};

template <int DT, bool SPARSE>
__device__ __forceinline__ void gload(StageRegs<DT, SPARSE>& r, const uint8_t* __restrict__ w,
                                      const uint32_t* __restrict__ meta,
                                      const uint8_t* __restrict__ x, int n0, int m0, int ks, int N,
                                      int M, int K, int tid) {
  using L = TiledLayout<DT, SPARSE>;
  using R = StageRegs<DT, SPARSE>;
  constexpr int WPR = L::WB / 16;  // pieces per W row
  const size_t wrow = SPARSE ? (size_t)(K / 2) * L::ESZ : (size_t)K * L::ESZ;
#pragma unroll
  for (int i = 0; i < R::WP; ++i) {
    const int p = tid + NT * i, row = p / WPR, c = p % WPR;
    int n = n0 + row;
    n = n < N ? n : N - 1;
    r.w[i] = *reinterpret_cast<const i32x4*>(w + (size_t)n * wrow + (size_t)ks * L::WB + 16 * c);
  }
  if constexpr (SPARSE) {
    int n = n0 + tid;
    n = n < N ? n : N - 1;
    const uint32_t* mp = meta + (size_t)n * (K / 32) + (size_t)ks * L::MWORDS;
    if constexpr (L::MWORDS == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(mp);
      r.meta[0] = v[0]; r.meta[1] = v[1]; r.meta[2] = v[2]; r.meta[3] = v[3];
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(mp);
      r.meta[0] = v[0]; r.meta[1] = v[1];
    }
  }
  const size_t xrow = (size_t)K * L::ESZ;
#pragma unroll
  for (int i = 0; i < R::XP; ++i) {
    const int p = tid + NT * i, row = p / 8, c = p % 8;
    int m = m0 + row;
    m = m < M ? m : M - 1;
    r.x[i] = *reinterpret_cast<const i32x4*>(x + (size_t)m * xrow + (size_t)ks * L::XB + 16 * c);
  }
}

template <int DT, bool SPARSE>
__device__ __forceinline__ void lstore(const StageRegs<DT, SPARSE>& r, uint8_t* __restrict__ buf,
                                       int tid) {
  using L = TiledLayout<DT, SPARSE>;
  using R = StageRegs<DT, SPARSE>;
  constexpr int WPR = L::WB / 16;
#pragma unroll
  for (int i = 0; i < R::WP; ++i) {
    const int p = tid + NT * i, row = p / WPR, c = p % WPR;
    *reinterpret_cast<i32x4*>(buf + L::W_OFF + row * L::WB + 16 * swz_w(row, c, WPR)) = r.w[i];
  }
  if constexpr (SPARSE) {
    if constexpr (L::MWORDS == 4)
      *reinterpret_cast<u32x4*>(buf + L::M_OFF + tid * 16) =
          u32x4{r.meta[0], r.meta[1], r.meta[2], r.meta[3]};
    else
      *reinterpret_cast<u32x2*>(buf + L::M_OFF + tid * 8) = u32x2{r.meta[0], r.meta[1]};
  }
#pragma unroll
  for (int i = 0; i < R::XP; ++i) {
    const int p = tid + NT * i, row = p / 8, c = p % 8;
    *reinterpret_cast<i32x4*>(buf + L::X_OFF + row * L::XB + 16 * swz_x(row, c)) = r.x[i];
  }
}

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// One K step from an LDS buffer: 2 substeps x 4 x 4 instructions per wave.
template <int DT, bool SPARSE>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[4][4], const uint8_t* __restrict__ buf,
                                         int wn, int wm, int lane) {
  using L = TiledLayout<DT, SPARSE>;
  constexpr int WPR = L::WB / 16;
  const int q = lane >> 5, r = lane & 31;
  constexpr int SUB = (SPARSE || DT == SP24_FP8_E4M3) ? 2 : 4;  // instructions along K per step
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    i32x4 a[4][SPARSE ? 1 : 2];
    uint32_t ix[4];
    i32x4 b[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wn * 128 + 32 * i + r;
      const uint8_t* wr = buf + L::W_OFF + row * L::WB;
      if constexpr (SPARSE) {
        // fp8: bytes [32s + 16q, +16) and word 2s + q; bf16: bytes [32q + 16s, +16), word q
        const int c = DT == SP24_FP8_E4M3 ? 2 * s + q : 2 * q + s;
        a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz_w(row, c, WPR));
        const int word = DT == SP24_FP8_E4M3 ? 2 * s + q : q;
        ix[i] = *reinterpret_cast<const uint32_t*>(buf + L::M_OFF + row * L::MWORDS * 4 + 4 * word);
      } else if constexpr (DT == SP24_FP8_E4M3) {
        // dense fp8: 32 bytes [64s + 32q, +32)
        a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz_w(row, 4 * s + 2 * q, WPR));
        a[i][1] = *reinterpret_cast<const i32x4*>(wr + 16 * swz_w(row, 4 * s + 2 * q + 1, WPR));
      } else {
        // dense bf16: 16 bytes [32s + 16q, +16)
        a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz_w(row, 2 * s + q, WPR));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wm * 128 + 32 * j + r;
      const uint8_t* xr = buf + L::X_OFF + row * L::XB;
      if constexpr (SPARSE) {
        // run h of lane group q: fp8 bytes 64s + 32h + 16q; bf16 bytes 64h + 32s + 16q
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = DT == SP24_FP8_E4M3 ? 4 * s + 2 * h + q : 4 * h + 2 * s + q;
          b[j][h] = *reinterpret_cast<const i32x4*>(xr + 16 * swz_x(row, c));
        }
      } else if constexpr (DT == SP24_FP8_E4M3) {
        b[j][0] = *reinterpret_cast<const i32x4*>(xr + 16 * swz_x(row, 4 * s + 2 * q));
        b[j][1] = *reinterpret_cast<const i32x4*>(xr + 16 * swz_x(row, 4 * s + 2 * q + 1));
      } else {
        b[j][0] = *reinterpret_cast<const i32x4*>(xr + 16 * swz_x(row, 2 * s + q));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (SPARSE && DT == SP24_FP8_E4M3) {
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a[i][0], cat8(b[j][0], b[j][1]),
                                                                   acc[i][j], (int)ix[i], 0, 0);
        } else if constexpr (SPARSE) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                __builtin_bit_cast(bf16x8, a[i][0]), __builtin_bit_cast(bf16x16, cat8(b[j][0], b[j][1])),
                acc[i][j], (int)ix[i], 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                __builtin_bit_cast(bf16x8, a[i][0]), __builtin_bit_cast(bf16x16, cat8(b[j][0], b[j][1])),
                acc[i][j], (int)ix[i], 0, 1);
        } else if constexpr (DT == SP24_FP8_E4M3) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              cat8(a[i][0], a[i][1]), cat8(b[j][0], b[j][1]), acc[i][j], 0, 0, 0, 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[i][0]), __builtin_bit_cast(bf16x8, b[j][0]), acc[i][j], 0, 0,
              0);
        }
      }
    }
  }
}

template <int DT, bool SPARSE>
__global__ __launch_bounds__(NT, 1) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, uint16_t* __restrict__ y,
    int M, int N, int K) {
  using L = TiledLayout<DT, SPARSE>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;

  // tile order: XCD-contiguous ranges, then groups of GROUP_N tile columns
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int total = tiles_n * tiles_m;
  int pid = blockIdx.x;
  if (total % 8 == 0) pid = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int per_group = GROUP_N * tiles_m;
  const int group = pid / per_group, first_n = group * GROUP_N;
  const int gsize = min(tiles_n - first_n, GROUP_N);
  const int tn = first_n + (pid % per_group) % gsize, tm = (pid % per_group) / gsize;
  const int n0 = tn * BN, m0 = tm * BM;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nks = K / L::KS;
  StageRegs<DT, SPARSE> st;
  gload<DT, SPARSE>(st, w, meta, x, n0, m0, 0, N, M, K, tid);
  lstore<DT, SPARSE>(st, lds, tid);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    uint8_t* cur = lds + (ks & 1) * L::STAGE;
    uint8_t* nxt = lds + ((ks + 1) & 1) * L::STAGE;
    const bool more = ks + 1 < nks;
    if (more) gload<DT, SPARSE>(st, w, meta, x, n0, m0, ks + 1, N, M, K, tid);
    mma_step<DT, SPARSE>(acc, cur, wn, wm, lane);
    if (more) lstore<DT, SPARSE>(st, nxt, tid);
    __syncthreads();
  }

  float scale = 1.0f;
  if constexpr (DT == SP24_FP8_E4M3) scale = x_scale[0] * w_scale[0];
  const int q = lane >> 5, c = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + 32 * j + c;
    if (m >= M) continue;
    uint16_t* yr = y + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 128 + 32 * i + 8 * g + 4 * q;  // registers 4g..4g+3: n .. n+3
        const uint32_t lo = f32_to_bf16_rne(acc[i][j][4 * g + 0] * scale) |
                            (f32_to_bf16_rne(acc[i][j][4 * g + 1] * scale) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[i][j][4 * g + 2] * scale) |
                            (f32_to_bf16_rne(acc[i][j][4 * g + 3] * scale) << 16);
        if (n + 3 < N && (N & 3) == 0) {
          *reinterpret_cast<u32x2*>(yr + n) = u32x2{lo, hi};
        } else {
          const uint32_t v[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yr[n + e] = (uint16_t)v[e];
        }
      }
    }
  }
}

template <int DT, bool SPARSE>
hipError_t launch_tiled_dt(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_tiled_kernel<DT, SPARSE>), dim3(p.grid_x), dim3(NT), 0, s,
                     static_cast<const uint8_t*>(a.x), static_cast<const uint8_t*>(a.w), a.meta,
                     a.x_scale, a.w_scale, a.y, a.m, a.n, a.k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  if (a.dtype == SP24_FP8_E4M3)
    return a.sparse ? launch_tiled_dt<SP24_FP8_E4M3, true>(a, p, s)
                    : launch_tiled_dt<SP24_FP8_E4M3, false>(a, p, s);
  return a.sparse ? launch_tiled_dt<SP24_BF16, true>(a, p, s) : launch_tiled_dt<SP24_BF16, false>(a, p, s);
}

}  // namespace sp24
