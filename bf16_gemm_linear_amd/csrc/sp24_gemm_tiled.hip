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
// of one, selected by abid (bf16).  INT8 takes the integer forms of the fp8
// instructions (v_smfmac_i32_32x32x64_i8; dense: two v_mfma_i32_32x32x32_i8)
// with the fp8 operand layouts; its int32 accumulators become fp32 before the
// epilogue.
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
#include <type_traits>

#include "sp24_common.hpp"
#include "sp24_dma.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

// Tile rows of W and of X.  This file is also compiled with SP24_TILED_BN = 128
// (sp24_gemm_tiled128.hip, one-byte codes only): 128 W rows x 256 tokens per
// workgroup, so that a one-token-tile product of a wide layer (gate+up at m = 256:
// 224 tiles) fills the chip.
#ifndef SP24_TILED_BN
#define SP24_TILED_BN 256
#define SP24_TILED_LAUNCH launch_gemm_tiled
#endif
constexpr int BN = SP24_TILED_BN, BM = 256;
constexpr int WGN = 2, WGM = 4;     // waves along n and along m
constexpr int NWAVES = WGN * WGM, NT = NWAVES * 64;
constexpr int TI = BN / WGN / 32;   // 32-row instruction tiles per wave along n
constexpr int TJ = BM / WGM / 32;   // 32-row instruction tiles per wave along m
constexpr int GROUP_N = 8;          // tile columns per group in the tile order

// K step and ring depth of the sparse one-byte kernels (the others keep
// one 128-byte X row segment per step and as many buffers as fit).
constexpr int kKsFp8Sparse = 128;
constexpr int kStagesFp8Sparse = 3;

template <int DT, bool SPARSE>
struct TiledLayout {
  static constexpr bool B8 = DT != SP24_BF16;  // one-byte codes (E4M3 or INT8)
  static constexpr int ESZ = B8 ? 1 : 2;
  static constexpr int KS = B8 ? (SPARSE ? kKsFp8Sparse : 128) : 64;  // K values per step
  static constexpr int WB = (SPARSE ? KS / 2 : KS) * ESZ;  // W bytes per row per step
  static constexpr int MWORDS = SPARSE ? KS / 32 : 0;     // metadata words per row per step
  static constexpr int XB = KS * ESZ;                      // X bytes per row per step
  static constexpr int WP = WB / 16, XP = XB / 16;        // 16-byte pieces per row
  static constexpr int W_OFF = 0;
  static constexpr int M_OFF = W_OFF + BN * WB;
  static constexpr int X_OFF = M_OFF + BN * MWORDS * 4;
  static constexpr int STAGE = X_OFF + BM * XB;           // bytes per LDS buffer
  static constexpr int STAGES = SPARSE ? (B8 ? kStagesFp8Sparse : 3) : 2;  // LDS buffers
  // 32x32 instructions along K per step: K 64 (sparse fp8, dense fp8), 32 (sparse bf16), 16 (dense bf16)
  static constexpr int SUB = KS / (B8 ? 64 : (SPARSE ? 32 : 16));
  static constexpr int YS = BN * 2 + 16;  // bytes per row of the output tile staged in LDS
  static constexpr int LDS_BYTES = STAGES * STAGE > BM * YS ? STAGES * STAGE : BM * YS;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Metadata of a row in an LDS buffer.  With 4 words per step (fp8), the
// words that lane group q needs for its two substeps (word q for substep 0,
// word q + 2 for substep 1) are adjacent: slot 2 * (q ^ ((r >> 4) & 1)) + s
// of row r holds word 2s + q, so one 8-byte read per row gives both, and the
// 32 rows of a half-wave read hit 64 distinct banks.  With 2 words per step
// (bf16) lane group q needs word q for both substeps, in slot q.
// meta_slot_word: the word of the step held by slot `slot` of row r.
template <int MWORDS>
__device__ __forceinline__ int meta_slot_word(int r, int slot) {
  if constexpr (MWORDS == 4) {
    const int q = (slot >> 1) ^ ((r >> 4) & 1), sub = slot & 1;
    return 2 * sub + q;
  } else {
    return slot;
  }
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
  size_t mblock;  // metadata words per 128-K block of all N rows

  // ks0: first K step of this workgroup's K slice (split-K; even, so that the
  // metadata offset of bf16's 2-word steps stays whole blocks of 4 words)
  __device__ __forceinline__ Loader(const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
                                    const uint8_t* __restrict__ x, int n0, int m0, int N, int M,
                                    int K, int wave_, int lane, int ks0 = 0)
      : wave(wave_), mblock((size_t)N * 4) {
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
        mp[j] = meta + (size_t)n * 4 + meta_slot_word<L::MWORDS>(row, p % L::MWORDS);
      }
    }
    const size_t xrow = (size_t)K * L::ESZ;
#pragma unroll
    for (int j = 0; j < S::X_INSTR; ++j) {
      const int p = (wave * S::X_INSTR + j) * 64 + lane, row = p / L::XP;
      const int m = min(m0 + row, M - 1);
      xp[j] = x + (size_t)m * xrow + 16 * swz16<L::XP>(row, p % L::XP);
    }
    if (ks0 != 0) {
#pragma unroll
      for (int j = 0; j < S::W_INSTR; ++j) wp[j] += (size_t)ks0 * L::WB;
      if constexpr (SPARSE) {
#pragma unroll
        for (int j = 0; j < S::M_INSTR; ++j) mp[j] += meta_step(ks0);
      }
#pragma unroll
      for (int j = 0; j < S::X_INSTR; ++j) xp[j] += (size_t)ks0 * L::XB;
    }
  }

  // Metadata of K step ks: its MWORDS words of every row sit at word (ks * MWORDS) % 4
  // of each row's 16 bytes in block (ks * MWORDS) / 4 (K % 128 == 0: whole blocks).
  __device__ __forceinline__ size_t meta_step(int ks) const {
    const int w0 = ks * L::MWORDS;
    return (size_t)(w0 >> 2) * mblock + (w0 & 3);
  }

  // Load J of this wave's share of K step ks (W pieces, then metadata words, then X pieces).
  template <int J>
  __device__ __forceinline__ void issue_one(uint8_t* buf, int ks) const {
    if constexpr (J < S::W_INSTR) {
      dma16(wp[J] + (size_t)ks * L::WB, buf + L::W_OFF + (wave * S::W_INSTR + J) * 1024);
    } else if constexpr (J < S::W_INSTR + S::M_INSTR) {
      constexpr int j = J - S::W_INSTR;
      dma4(mp[j] + meta_step(ks), buf + L::M_OFF + (wave * S::M_INSTR + j) * 256);
    } else {
      constexpr int j = J - S::W_INSTR - S::M_INSTR;
      dma16(xp[j] + (size_t)ks * L::XB, buf + L::X_OFF + (wave * S::X_INSTR + j) * 1024);
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
        dma4(mp[j] + meta_step(ks), buf + L::M_OFF + (wave * S::M_INSTR + j) * 256);
    }
#pragma unroll
    for (int j = 0; j < S::X_INSTR; ++j)
      dma16(xp[j] + (size_t)ks * L::XB, buf + L::X_OFF + (wave * S::X_INSTR + j) * 1024);
  }
};

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operands of one substep (one instruction along K) for a wave's TI x TJ
// instruction tiles.
template <int DT, bool SPARSE>
struct Frag {
  i32x4 a[TI][SPARSE ? 1 : 2];
  uint32_t ix[TI];   // index bits of this substep
  uint32_t ixn[TI];  // index bits of the next substep of the same step (read together)
  i32x4 b[TJ][2];
};

// Reads of one substep, numbered: A operands (one per instruction row i),
// then X runs (two per instruction column j), then metadata words (one per i).
template <bool SPARSE>
constexpr int n_pieces() {
  return TI + 2 * TJ + (SPARSE ? TI : 0);
}

// Read piece P of substep s from an LDS buffer into f.
template <int DT, bool SPARSE, int P>
__device__ __forceinline__ void read_piece(Frag<DT, SPARSE>& f, const Frag<DT, SPARSE>& prev,
                                           const uint8_t* __restrict__ buf, int s, int wn, int wm, int lane) {
  using L = TiledLayout<DT, SPARSE>;
  const int q = lane >> 5, r = lane & 31;
  if constexpr (P < TI) {
    constexpr int i = P;
    const int row = wn * (BN / WGN) + 32 * i + r;
    const uint8_t* wr = buf + L::W_OFF + row * L::WB;
    if constexpr (SPARSE) {
      // fp8: bytes [32s + 16q, +16); bf16: bytes [32q + 16s, +16)
      const int c = DT != SP24_BF16 ? 2 * s + q : 2 * q + s;
      f.a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, c));
    } else if constexpr (DT != SP24_BF16) {
      // dense fp8, int8: 32 bytes [64s + 32q, +32)
      f.a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 4 * s + 2 * q));
      f.a[i][1] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 4 * s + 2 * q + 1));
    } else {
      // dense bf16: 16 bytes [32s + 16q, +16)
      f.a[i][0] = *reinterpret_cast<const i32x4*>(wr + 16 * swz16<L::WP>(row, 2 * s + q));
    }
  } else if constexpr (P < TI + 2 * TJ) {
    constexpr int j = (P - TI) / 2, h = (P - TI) % 2;
    const int row = wm * (BM / WGM) + 32 * j + r;
    const uint8_t* xr = buf + L::X_OFF + row * L::XB;
    if constexpr (SPARSE) {
      // run h of lane group q: fp8 bytes 64s + 32h + 16q; bf16 bytes 64h + 32s + 16q
      const int c = DT != SP24_BF16 ? 4 * s + 2 * h + q : 4 * h + 2 * s + q;
      f.b[j][h] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, c));
    } else if constexpr (DT != SP24_BF16) {
      f.b[j][h] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, 4 * s + 2 * q + h));
    } else if constexpr (h == 0) {
      f.b[j][0] = *reinterpret_cast<const i32x4*>(xr + 16 * swz16<L::XP>(row, 2 * s + q));
    }
  } else {
    // index bits: fp8 word 2s + q; bf16 word q (its 16-bit half s is selected by
    // abid).  Substep 0 reads both substeps' words; substep 1 takes them over.
    static_assert(L::SUB == 2, "two substeps per step in the sparse kernels");
    constexpr int i = P - TI - 2 * TJ;
    if (s == 0) {
      const int row = wn * (BN / WGN) + 32 * i + r;
      if constexpr (DT != SP24_BF16) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(buf + L::M_OFF + row * 16 +
                                                        8 * (q ^ ((row >> 4) & 1)));
        f.ix[i] = v[0];
        f.ixn[i] = v[1];
      } else {
        f.ix[i] = *reinterpret_cast<const uint32_t*>(buf + L::M_OFF + row * 8 + 4 * q);
        f.ixn[i] = f.ix[i];
      }
    } else {
      f.ix[i] = prev.ixn[i];
    }
  }
}

template <int DT, bool SPARSE, int P0, int P1>
__device__ __forceinline__ void read_pieces(Frag<DT, SPARSE>& f, const Frag<DT, SPARSE>& prev,
                                            const uint8_t* __restrict__ buf, int s, int wn, int wm, int lane) {
  if constexpr (P0 < P1) {
    read_piece<DT, SPARSE, P0>(f, prev, buf, s, wn, wm, lane);
    read_pieces<DT, SPARSE, P0 + 1, P1>(f, prev, buf, s, wn, wm, lane);
  }
}

template <int DT, bool SPARSE, int J0, int J1>
__device__ __forceinline__ void issue_loads(const Loader<DT, SPARSE>& ld, uint8_t* buf, int ks) {
  if constexpr (J0 < J1) {
    ld.template issue_one<J0>(buf, ks);
    issue_loads<DT, SPARSE, J0 + 1, J1>(ld, buf, ks);
  }
}

// Matrix instruction (I, J) of substep S.
template <int DT, bool SPARSE, int S, int I, int J>
__device__ __forceinline__ void mma_one(f32x16 (&acc)[TI][TJ], const Frag<DT, SPARSE>& f) {
  if constexpr (SPARSE && DT == SP24_INT8) {
    acc[I][J] = __builtin_bit_cast(f32x16, __builtin_amdgcn_smfmac_i32_32x32x64_i8(
                                               f.a[I][0], cat8(f.b[J][0], f.b[J][1]),
                                               __builtin_bit_cast(i32x16, acc[I][J]), (int)f.ix[I], 0, 0));
  } else if constexpr (SPARSE && DT == SP24_FP8_E4M3) {
    acc[I][J] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(f.a[I][0], cat8(f.b[J][0], f.b[J][1]), acc[I][J],
                                                             (int)f.ix[I], 0, 0);
  } else if constexpr (SPARSE) {
    acc[I][J] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
        __builtin_bit_cast(bf16x8, f.a[I][0]), __builtin_bit_cast(bf16x16, cat8(f.b[J][0], f.b[J][1])),
        acc[I][J], (int)f.ix[I], 0, S & 1);
  } else if constexpr (DT == SP24_INT8) {
    // dense INT8: two instructions of K=32 over the lane group's 32 bytes
    acc[I][J] = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                               f.a[I][0], f.b[J][0], __builtin_bit_cast(i32x16, acc[I][J]), 0, 0, 0));
    acc[I][J] = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                               f.a[I][1], f.b[J][1], __builtin_bit_cast(i32x16, acc[I][J]), 0, 0, 0));
  } else if constexpr (DT == SP24_FP8_E4M3) {
    acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat8(f.a[I][0], f.a[I][1]),
                                                                cat8(f.b[J][0], f.b[J][1]), acc[I][J], 0, 0,
                                                                0, 0, 0, 0);
  } else {
    acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[I][0]),
                                                        __builtin_bit_cast(bf16x8, f.b[J][0]), acc[I][J], 0,
                                                        0, 0);
  }
}

// One substep's matrix instructions from `cur`, each followed by its share of
// the reads of the next substep (into `nxt`, substep `rs` of `rbuf`) and, with
// ISSUE, of the global->LDS loads of step `fill_ks` into `fill`.  The order is
// fixed (scheduling barriers), so every wave starts its matrix instructions
// at once and no wave issues a long burst of LDS reads that would stall its
// own matrix instructions behind a full LDS queue.
template <int DT, bool SPARSE, int S, int T, bool ISSUE>
__device__ __forceinline__ void phase(f32x16 (&acc)[TI][TJ], const Frag<DT, SPARSE>& cur, Frag<DT, SPARSE>& nxt,
                                      const uint8_t* __restrict__ rbuf, int rs, int wn, int wm, int lane,
                                      const Loader<DT, SPARSE>& ld, uint8_t* fill, int fill_ks) {
  constexpr int NMMA = TI * TJ, NP = n_pieces<SPARSE>();
  constexpr int NV = ISSUE ? StageLoads<DT, SPARSE>::TOTAL : 0;
  // the reads go out with the first RS instructions, so the last ones cover
  // their latency before the wait at the end of the phase
  constexpr int RS = NMMA > 4 ? NMMA - 3 : NMMA;
  if constexpr (T < NMMA) {
    mma_one<DT, SPARSE, S, T / TJ, T % TJ>(acc, cur);
    issue_loads<DT, SPARSE, T * NV / NMMA, (T + 1) * NV / NMMA>(ld, fill, fill_ks);
    if constexpr (T < RS) read_pieces<DT, SPARSE, T * NP / RS, (T + 1) * NP / RS>(nxt, cur, rbuf, rs, wn, wm, lane);
    __builtin_amdgcn_sched_barrier(0);
    phase<DT, SPARSE, S, T + 1, ISSUE>(acc, cur, nxt, rbuf, rs, wn, wm, lane, ld, fill, fill_ks);
  }
}

// Substeps S .. SUB-2 of a K step: substep S + 1 is read while substep S is
// multiplied.
template <int DT, bool SPARSE, int S>
__device__ __forceinline__ void inner_substeps(f32x16 (&acc)[TI][TJ], Frag<DT, SPARSE> (&f)[2],
                                               const uint8_t* __restrict__ cur, int wn, int wm, int lane,
                                               const Loader<DT, SPARSE>& ld) {
  using L = TiledLayout<DT, SPARSE>;
  if constexpr (S + 1 < L::SUB) {
    // The reads of substep S (issued a phase earlier) are done; waiting here,
    // before the next reads go out, lets the matrix instructions start
    // without waiting for those.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    phase<DT, SPARSE, S, 0, false>(acc, f[S & 1], f[(S + 1) & 1], cur, S + 1, wn, wm, lane, ld, nullptr, 0);
    inner_substeps<DT, SPARSE, S + 1>(acc, f, cur, wn, wm, lane, ld);
  }
}

// PARTIAL (split-K): workgroup (tile, blockIdx.y) multiplies K steps
// [blockIdx.y * slice_steps, +slice_steps) and writes its fp32 tile, unscaled, to
// partial[blockIdx.y][m][n]; the reduction applies the scales.
// ROWS: the tile's W rows (BN), part of the kernel's name so that traces tell the
// two tile shapes apart.
template <int DT, bool SPARSE, bool PARTIAL, int ROWS>
__global__ __launch_bounds__(NT, 2) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, uint16_t* __restrict__ y,
    int M, int N, int K, int xs_step, int ws_step, float* __restrict__ partial, int slice_steps) {
  static_assert(ROWS == BN, "the tile rows of this build");
  using L = TiledLayout<DT, SPARSE>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::LDS_BYTES];

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

  // STAGES LDS buffers in a ring, K step ks in buffer ks % STAGES, and two
  // register sets of operands, so LDS reads, global->LDS loads and matrix
  // instructions overlap.  Within step ks, substep s + 1 is read while
  // substep s is multiplied.  Before the last substep's instructions each
  // wave waits for its own loads of step ks + 1 and for its LDS reads of step
  // ks; the barrier after that makes every wave's loads of step ks + 1 visible
  // and guarantees that no wave still reads buffer ks % STAGES, which then
  // receives the loads of step ks + STAGES while the last substep's
  // instructions run and substep 0 of step ks + 1 is read.
  //
  // The barrier is a bare s_barrier: __syncthreads() adds a workgroup release
  // fence, which would wait for every outstanding LDS-DMA load (vmcnt(0)) and
  // drain the ring; the explicit counter waits provide the ordering.
  constexpr int STAGES = L::STAGES, SUB = L::SUB;
  constexpr int PER_STEP = StageLoads<DT, SPARSE>::TOTAL;
  const int nks = PARTIAL ? slice_steps : K / L::KS;
  const Loader<DT, SPARSE> ld(w, meta, x, n0, m0, N, M, K, wave, lane, PARTIAL ? (int)blockIdx.y * slice_steps : 0);
#pragma unroll
  for (int p = 0; p < STAGES; ++p)
    if (p < nks) ld.issue(lds + p * L::STAGE, p);
  wait_later<PER_STEP, STAGES - 1>(min(nks - 1, STAGES - 1));  // step 0 has landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frag<DT, SPARSE> f[2];
  read_pieces<DT, SPARSE, 0, n_pieces<SPARSE>()>(f[0], f[1], lds, 0, wn, wm, lane);

  // One K step.  ISSUE: step ks + STAGES exists and is loaded here.
  auto step = [&](int ks, auto issue_tag) {
    constexpr bool ISSUE = decltype(issue_tag)::value;
    const uint8_t* cur = lds + (ks % STAGES) * L::STAGE;
    inner_substeps<DT, SPARSE, 0>(acc, f, cur, wn, wm, lane, ld);
    // loads issued after those of step ks + 1: steps ks+2 .. ks+STAGES-1 (when they exist)
    if constexpr (ISSUE) {
      wait_vmcnt<(STAGES - 2) * PER_STEP>();
    } else {
      wait_later<PER_STEP, STAGES - 2>(max(0, min(nks - 2 - ks, STAGES - 2)));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of step ks are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // The last substep, the reads of substep 0 of step ks + 1 (after the last
    // step: a harmless read of a valid buffer) and the loads of step ks + STAGES.
    phase<DT, SPARSE, SUB - 1, 0, ISSUE>(acc, f[(SUB - 1) & 1], f[0], lds + ((ks + 1) % STAGES) * L::STAGE, 0,
                                         wn, wm, lane, ld, lds + (ks % STAGES) * L::STAGE, ks + STAGES);
  };
  const int nissue = max(0, nks - STAGES);
  for (int ks = 0; ks < nissue; ++ks) step(ks, std::true_type{});
  for (int ks = nissue; ks < nks; ++ks) step(ks, std::false_type{});

  // Epilogue through LDS.  Each accumulator register holds one output of a
  // 32-row column strip, so direct stores would send 8-byte pieces of 32
  // different rows per instruction; instead the tile is staged in LDS (the
  // ring is free: the last step waited for every load, and the barrier below
  // waits for every wave's last reads) and written back as whole rows, 16
  // bytes per lane.  Rows of the staged tile are padded by 16 bytes so the
  // 8-byte writes of a 32-row strip spread over the banks.
  constexpr int YS = L::YS;
  static_assert(BM * YS <= L::LDS_BYTES, "staged output tile fits");
  if constexpr (PARTIAL) {
    // fp32 partial tile straight from the accumulators: register 4g + e of tile
    // (i, j) holds row ml, columns nl + e (e < 4)
    if constexpr (DT == SP24_INT8)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = i32_bits_to_f32(acc[i][j][e]);
    const int q = lane >> 5, c = lane & 31;
    float* pz = partial + (size_t)blockIdx.y * M * N;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * (BM / WGM) + 32 * j + c;
      if (m >= M) continue;
      float* pr = pz + (size_t)m * N;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * (BN / WGN) + 32 * i + 8 * g + 4 * q;
          const f32x4 v = f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<f32x4*>(pr + n) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) pr[n + e] = v[e];
          }
        }
    }
    return;
  }
  if constexpr (DT == SP24_INT8)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = i32_bits_to_f32(acc[i][j][e]);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's last (discarded) reads are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  {
    const int q = lane >> 5, c = lane & 31;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int ml = wm * (BM / WGM) + 32 * j + c;
      // FP8, INT8: fp32(sx * sw) with the scales of X row m0 + ml and W row n (one per
      // tensor: step 0; rows past M or N are staged but never stored)
      float sx = 1.0f;
      if constexpr (DT != SP24_BF16) sx = x_scale[(size_t)min(m0 + ml, M - 1) * xs_step];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // accumulator registers 4g..4g+3 hold columns nl .. nl+3 of row ml
          const int nl = wn * (BN / WGN) + 32 * i + 8 * g + 4 * q;
          float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
          if constexpr (DT != SP24_BF16) {
            if (ws_step == 0) {  // one W scale per tensor: the common case, one product per row
              sc[0] = sc[1] = sc[2] = sc[3] = sx * w_scale[0];
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[e] = sx * w_scale[(size_t)min(n0 + nl + e, N - 1) * ws_step];
            }
          }
          const uint32_t lo = f32_to_bf16_rne(acc[i][j][4 * g + 0] * sc[0]) |
                              (f32_to_bf16_rne(acc[i][j][4 * g + 1] * sc[1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc[i][j][4 * g + 2] * sc[2]) |
                              (f32_to_bf16_rne(acc[i][j][4 * g + 3] * sc[3]) << 16);
          *reinterpret_cast<u32x2*>(lds + ml * YS + nl * 2) = u32x2{lo, hi};
        }
      }
    }
  }
  __syncthreads();
  // 32 lanes per row, 8 columns (16 bytes) per lane, two rows per wave per pass
  constexpr int LPR = BN / 8;           // lanes per row
  constexpr int RPP = 64 / LPR;         // rows per wave per pass
  const int nl = 8 * (lane % LPR);
  const int n = n0 + nl;
  const bool vec = (N & 7) == 0 && n + 7 < N;
#pragma unroll 4
  for (int r0 = wave * RPP; r0 < BM; r0 += NWAVES * RPP) {
    const int ml = r0 + lane / LPR;
    const int m = m0 + ml;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + ml * YS + nl * 2);
    if (m >= M) continue;
    uint16_t* yr = y + (size_t)m * N;
    if (vec) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(yr + n));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) yr[n + e] = (uint16_t)(v[e / 2] >> (16 * (e & 1)));
    }
  }
}

template <int DT, bool SPARSE>
hipError_t launch_tiled_dt(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  using L = TiledLayout<DT, SPARSE>;
  if (p.split_k > 1)
    hipLaunchKernelGGL((gemm_tiled_kernel<DT, SPARSE, true, BN>), dim3(p.grid_x, p.split_k), dim3(NT), 0, s,
                       static_cast<const uint8_t*>(a.x), static_cast<const uint8_t*>(a.w), a.meta, a.x_scale,
                       a.w_scale, a.y, a.m, a.n, a.k, a.x_scale_step, a.w_scale_step, a.partial,
                       a.k / L::KS / p.split_k);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<DT, SPARSE, false, BN>), dim3(p.grid_x), dim3(NT), 0, s,
                       static_cast<const uint8_t*>(a.x), static_cast<const uint8_t*>(a.w), a.meta, a.x_scale,
                       a.w_scale, a.y, a.m, a.n, a.k, a.x_scale_step, a.w_scale_step, (float*)nullptr, 0);
  return hipGetLastError();
}

}  // namespace

hipError_t SP24_TILED_LAUNCH(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  if (a.dtype == SP24_FP8_E4M3)
    return a.sparse ? launch_tiled_dt<SP24_FP8_E4M3, true>(a, p, s)
                    : launch_tiled_dt<SP24_FP8_E4M3, false>(a, p, s);
  if (a.dtype == SP24_INT8)
    return a.sparse ? launch_tiled_dt<SP24_INT8, true>(a, p, s) : launch_tiled_dt<SP24_INT8, false>(a, p, s);
#if SP24_TILED_BN == 256
  return a.sparse ? launch_tiled_dt<SP24_BF16, true>(a, p, s) : launch_tiled_dt<SP24_BF16, false>(a, p, s);
#else
  // bf16 metadata steps (two words per row) do not split over 8 waves at 128 rows
  return hipErrorInvalidConfiguration;
#endif
}

}  // namespace sp24
