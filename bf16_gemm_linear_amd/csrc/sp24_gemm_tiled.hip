// Large-m ("prefill") GEMM kernels: Y[m, n] = sum_k X[m, k] W[n, k] with
// 256 x 256 output tiles per workgroup, staged through LDS.
//
// At prefill sizes the product is bound by matrix-core throughput.  Each
// workgroup (8 waves, two per SIMD) owns a 256 (n) x 256 (m) tile of Y and
// walks K in steps of KS = 128 (fp8) or 64 (bf16) values.  A step brings, for
// every W row, 64 bytes of compressed values plus KS/32 metadata words (dense
// baseline: 128 bytes of values), and for every X row 128 bytes.  Operands go
// from global memory straight into a ring of LDS buffers with
// global_load_lds (3 buffers for the sparse kernels, so the loads of steps k+1
// and k+2 are in flight while step k is multiplied; 2 for the dense baseline,
// whose W tile is twice as large).  Each wave computes a 128 (n) x 64 (m)
// sub-tile as 4 x 2 instructions of 32 x 32 (sparse:
// v_smfmac_f32_32x32x64_fp8_fp8 / v_smfmac_f32_32x32x32_bf16; dense baseline:
// v_mfma_f32_32x32x64_f8f6f4 / v_mfma_f32_32x32x16_bf16).
//
// Operand layouts of the 32x32 sparse instructions (measured on gfx950 with
// one-hot probes): A lane l holds W row l%32 and, for lane group q = l/32,
// the contiguous instruction-K half [q*Kt/2, (q+1)*Kt/2) with its index bits;
// B lane l holds X row l%32 and two runs of Kt/4 values, run h covering
// instruction K [h*Kt/2 + q*Kt/4, ...).  Instruction K is mapped to the
// step's K so that every operand of a lane is one 16-byte piece of its row
// and the index bits of a lane are one metadata word (fp8) or one 16-bit half
// of one, selected by abid (bf16).
//
// LDS rows are XOR-swizzled in 16-byte units (and metadata words within a
// row) so that the operand reads of a wave spread over the banks; the LDS-DMA
// load writes lane i's bytes to slot i of a 1 KB block, so the swizzle is
// applied on the global side (XOR swizzles are their own inverse) and every
// load instruction still reads whole 64- or 128-byte row segments.
// (A fragment-major LDS order -- one contiguous block per operand read --
// measured slower: its loads gather 32-byte pieces.)  Workgroups are mapped to
// tiles XCD by XCD and, inside an XCD, in groups of 8 tile columns, so that
// workgroups resident at the same time share W and X tiles in their XCD's L2.
#include "sp24_common.hpp"
#include "sp24_dma.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int BN = 256, BM = 256;  // tile rows of W and of X
constexpr int WGN = 2, WGM = 4;     // waves along n and along m
constexpr int NWAVES = WGN * WGM, NT = NWAVES * 64;
constexpr int TI = BN / WGN / 32;   // 32-row instruction tiles per wave along n
constexpr int TJ = BM / WGM / 32;   // 32-row instruction tiles per wave along m
constexpr int GROUP_N = 8;          // tile columns per group in the tile order

// K step and ring depth of the sparse FP8 kernel (the other three keep
// one 128-byte X row segment per step and as many buffers as fit).
constexpr int kKsFp8Sparse = 128;
constexpr int kStagesFp8Sparse = 3;

template <int DT, bool SPARSE>
struct TiledLayout {
  static constexpr bool FP8 = DT == SP24_FP8_E4M3;
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int KS = FP8 ? (SPARSE ? kKsFp8Sparse : 128) : 64;  // K values per step
  static constexpr int WB = (SPARSE ? KS / 2 : KS) * ESZ;  // W bytes per row per step
  static constexpr int MWORDS = SPARSE ? KS / 32 : 0;     // metadata words per row per step
  static constexpr int XB = KS * ESZ;                      // X bytes per row per step
  static constexpr int WP = WB / 16, XP = XB / 16;        // 16-byte pieces per row
  static constexpr int W_OFF = 0;
  static constexpr int M_OFF = W_OFF + BN * WB;
  static constexpr int X_OFF = M_OFF + BN * MWORDS * 4;
  static constexpr int STAGE = X_OFF + BM * XB;           // bytes per LDS buffer
  static constexpr int STAGES = SPARSE ? (FP8 ? kStagesFp8Sparse : 3) : 2;  // LDS buffers
  // 32x32 instructions along K per step: K 64 (sparse fp8, dense fp8), 32 (sparse bf16), 16 (dense bf16)
  static constexpr int SUB = KS / (FP8 ? 64 : (SPARSE ? 32 : 16));
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS budget");
};

// Metadata words of a row (MWORDS per row): with 4 words, word w of row r sits
// at w ^ (2 * ((r >> 4) & 1)), so the 64 lanes of a read (32 rows x words 2s,
// 2s+1) hit 64 distinct banks; with 2 words a read is already contiguous.
__device__ __forceinline__ int swz_m(int row, int w, int words) {
  return words == 4 ? (w ^ (((row >> 4) & 1) * 2)) : w;
}

template <int DT, bool SPARSE>
struct StageLoads {
  using L = TiledLayout<DT, SPARSE>;
  static constexpr int W_INSTR = BN * L::WB / 1024 / NWAVES;     // per wave
  static constexpr int X_INSTR = BM * L::XB / 1024 / NWAVES;
  static constexpr int M_INSTR = SPARSE ? BN * L::MWORDS / 64 / NWAVES : 0;  // dword loads
  static_assert(W_INSTR * 1024 * NWAVES == BN * L::WB, "W pieces split evenly");
  static_assert(X_INSTR * 1024 * NWAVES == BM * L::XB, "X pieces split evenly");
  static_assert(!SPARSE || M_INSTR * 64 * NWAVES == BN * L::MWORDS, "metadata words split evenly");
  static constexpr int TOTAL = W_INSTR + X_INSTR + M_INSTR;  // VMEM instructions per wave per step
};

// Per-lane source pointers of this wave's share of step 0; step ks adds ks
// times the bytes per step.  Instruction j of wave w fills LDS slots
// [(w * INSTR + j) * 64, +64) of its region; slot p holds (row p / pieces,
// piece swz(row, p % pieces)).
template <int DT, bool SPARSE>
struct Loader {
  using L = TiledLayout<DT, SPARSE>;
  using S = StageLoads<DT, SPARSE>;
  const uint8_t* wp[S::W_INSTR];
  const uint32_t* mp[S::M_INSTR > 0 ? S::M_INSTR : 1];
  const uint8_t* xp[S::X_INSTR];
  int wave;  // wave-uniform (scalar)

  __device__ __forceinline__ Loader(const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
                                    const uint8_t* __restrict__ x, int n0, int m0, int N, int M,
                                    int K, int wave_, int lane)
      : wave(wave_) {
    const size_t wrow = SPARSE ? (size_t)(K / 2) * L::ESZ : (size_t)K * L::ESZ;
#pragma unroll
    for (int j = 0; j < S::W_INSTR; ++j) {
      const int p = (wave * S::W_INSTR + j) * 64 + lane, row = p / L::WP;
      const int n = min(n0 + row, N - 1);  // ragged n: clamp the load, the store is masked
      wp[j] = w + (size_t)n * wrow + 16 * swz16<L::WP>(row, p % L::WP);
    }
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < S::M_INSTR; ++j) {
        const int p = (wave * S::M_INSTR + j) * 64 + lane, row = p / L::MWORDS;
        const int n = min(n0 + row, N - 1);
        mp[j] = meta + (size_t)n * (K / 32) + swz_m(row, p % L::MWORDS, L::MWORDS);
      }
    }
    const size_t xrow = (size_t)K * L::ESZ;
#pragma unroll
    for (int j = 0; j < S::X_INSTR; ++j) {
      const int p = (wave * S::X_INSTR + j) * 64 + lane, row = p / L::XP;
      const int m = min(m0 + row, M - 1);
      xp[j] = x + (size_t)m * xrow + 16 * swz16<L::XP>(row, p % L::XP);
    }
  }

  // Issue every load of K step ks into the LDS buffer `buf`.
  __device__ __forceinline__ void issue(uint8_t* buf, int ks) const {
#pragma unroll
    for (int j = 0; j < S::W_INSTR; ++j)
      dma16(wp[j] + (size_t)ks * L::WB, buf + L::W_OFF + (wave * S::W_INSTR + j) * 1024);
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < S::M_INSTR; ++j)
        dma4(mp[j] + (size_t)ks * L::MWORDS, buf + L::M_OFF + (wave * S::M_INSTR + j) * 256);
    }
#pragma unroll
    for (int j = 0; j < S::X_INSTR; ++j)
      dma16(xp[j] + (size_t)ks * L::XB, buf + L::X_OFF + (wave * S::X_INSTR + j) * 1024);
  }
};

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Scheduling groups: N times (A matrix instructions, then B vector-memory
// instructions), so the loads of a later step issue between matrix
// instructions instead of in one burst that stalls the wave.
template <int N, int A, int B>
__device__ __forceinline__ void interleave_groups() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, B, 0);
    interleave_groups<N - 1, A, B>();
  }
}

// One K step from an LDS buffer: SUB substeps x TI x TJ instructions per wave.
// Every operand of the step is read from LDS first and a scheduling barrier
// keeps the compiler from interleaving (and serialising) reads and matrix
// instructions, so the reads of later substeps overlap the first instructions.
// With ISSUE, the loads of step `nxt` into `nbuf` are issued interleaved with
// the matrix instructions.
template <int DT, bool SPARSE, bool ISSUE>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[TI][TJ], const uint8_t* __restrict__ buf,
                                         int wn, int wm, int lane, const Loader<DT, SPARSE>& ld,
                                         uint8_t* nbuf, int nxt) {
  using L = TiledLayout<DT, SPARSE>;
  constexpr int SUB = L::SUB;
  const int q = lane >> 5, r = lane & 31;
  i32x4 a[SUB][TI][SPARSE ? 1 : 2];
  uint32_t ix[SUB][TI];
  i32x4 b[SUB][TJ][2];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wn * (BN / WGN) + 32 * i + r;
      const uint8_t* wr = buf + L::W_OFF + row * L::WB;
      if constexpr (SPARSE) {
        // fp8: bytes [32s + 16q, +16) and word 2s + q; bf16: bytes [32q + 16s, +16),
        // word q (its 16-bit half s is selected by abid)
        const int c = DT == SP24_FP8_E4M3 ? 2 * s + q : 2 * q + s;
        a[s][i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, c));
        const int word = DT == SP24_FP8_E4M3 ? 2 * s + q : q;
        ix[s][i] = *reinterpret_cast<const uint32_t*>(buf + L::M_OFF + row * L::MWORDS * 4 +
                                                      4 * swz_m(row, word, L::MWORDS));
      } else if constexpr (DT == SP24_FP8_E4M3) {
        // dense fp8: 32 bytes [64s + 32q, +32)
        a[s][i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 4 * s + 2 * q));
        a[s][i][1] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 4 * s + 2 * q + 1));
      } else {
        // dense bf16: 16 bytes [32s + 16q, +16)
        a[s][i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 2 * s + q));
      }
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wm * (BM / WGM) + 32 * j + r;
      const uint8_t* xr = buf + L::X_OFF + row * L::XB;
      if constexpr (SPARSE) {
        // run h of lane group q: fp8 bytes 64s + 32h + 16q; bf16 bytes 64h + 32s + 16q
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = DT == SP24_FP8_E4M3 ? 4 * s + 2 * h + q : 4 * h + 2 * s + q;
          b[s][j][h] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, c));
        }
      } else if constexpr (DT == SP24_FP8_E4M3) {
        b[s][j][0] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, 4 * s + 2 * q));
        b[s][j][1] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, 4 * s + 2 * q + 1));
      } else {
        b[s][j][0] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, 2 * s + q));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (ISSUE) ld.issue(nbuf, nxt);
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (SPARSE && DT == SP24_FP8_E4M3) {
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(
              a[s][i][0], cat8(b[s][j][0], b[s][j][1]), acc[i][j], (int)ix[s][i], 0, 0);
        } else if constexpr (SPARSE) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                __builtin_bit_cast(bf16x8, a[s][i][0]),
                __builtin_bit_cast(bf16x16, cat8(b[s][j][0], b[s][j][1])), acc[i][j], (int)ix[s][i], 0,
                0);
          else
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                __builtin_bit_cast(bf16x8, a[s][i][0]),
                __builtin_bit_cast(bf16x16, cat8(b[s][j][0], b[s][j][1])), acc[i][j], (int)ix[s][i], 0,
                1);
        } else if constexpr (DT == SP24_FP8_E4M3) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              cat8(a[s][i][0], a[s][i][1]), cat8(b[s][j][0], b[s][j][1]), acc[i][j], 0, 0, 0, 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[s][i][0]), __builtin_bit_cast(bf16x8, b[s][j][0]), acc[i][j],
              0, 0, 0);
        }
      }
    }
  }
  if constexpr (ISSUE) {
    constexpr int NMMA = SUB * TI * TJ, NLD = StageLoads<DT, SPARSE>::TOTAL;
    interleave_groups<NLD, NMMA / NLD, 1>();
    if constexpr (NMMA % NLD != 0) __builtin_amdgcn_sched_group_barrier(0x008, NMMA % NLD, 0);
  }
}

template <int DT, bool SPARSE>
__global__ __launch_bounds__(NT, 2) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, uint16_t* __restrict__ y,
    int M, int N, int K) {
  using L = TiledLayout<DT, SPARSE>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::STAGES * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS destinations stay in SGPRs
  const int wn = wave / WGM, wm = wave % WGM;

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

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // STAGES LDS buffers in a ring.  At the top of step ks a wave waits for its
  // own loads of step ks, the barrier makes every wave's loads visible (and
  // guarantees every wave is done reading buffer (ks - 1) % STAGES), and then
  // the loads of step ks + STAGES - 1 go into that buffer while step ks is
  // multiplied.
  constexpr int STAGES = L::STAGES;
  constexpr int PER_STEP = StageLoads<DT, SPARSE>::TOTAL;
  const int nks = K / L::KS;
  const Loader<DT, SPARSE> ld(w, meta, x, n0, m0, N, M, K, wave, lane);
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < nks) ld.issue(lds + p * L::STAGE, p);
  // steps whose loop issues the loads of step ks + STAGES - 1, then the last ones
  const int nissue = max(0, nks - (STAGES - 1));
  for (int ks = 0; ks < nissue; ++ks) {
    wait_vmcnt<(STAGES - 2) * PER_STEP>();  // loads of steps ks+1 .. ks+STAGES-2 may be in flight
    __builtin_amdgcn_s_barrier();
    const int nxt = ks + STAGES - 1;
    mma_step<DT, SPARSE, true>(acc, lds + (ks % STAGES) * L::STAGE, wn, wm, lane, ld,
                               lds + (nxt % STAGES) * L::STAGE, nxt);
  }
  for (int ks = nissue; ks < nks; ++ks) {
    // loads issued after those of step ks: steps ks+1 .. ks+STAGES-2 (when they exist)
    wait_later<PER_STEP, STAGES - 2>(min(nks - 1 - ks, STAGES - 2));
    // A bare barrier: __syncthreads() adds a workgroup release fence, which
    // would wait for every outstanding LDS-DMA load (vmcnt(0)) and drain the
    // pipeline.  The explicit vmcnt wait above already covers step ks, and each
    // wave's LDS reads of the previous step completed before their results
    // fed its matrix instructions.
    __builtin_amdgcn_s_barrier();
    mma_step<DT, SPARSE, false>(acc, lds + (ks % STAGES) * L::STAGE, wn, wm, lane, ld, nullptr, 0);
  }

  float scale = 1.0f;
  if constexpr (DT == SP24_FP8_E4M3) scale = x_scale[0] * w_scale[0];
  const int q = lane >> 5, c = lane & 31;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = m0 + wm * (BM / WGM) + 32 * j + c;
    if (m >= M) continue;
    uint16_t* yr = y + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // accumulator registers 4g..4g+3 hold rows n .. n+3 of this column
        const int n = n0 + wn * (BN / WGN) + 32 * i + 8 * g + 4 * q;
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
