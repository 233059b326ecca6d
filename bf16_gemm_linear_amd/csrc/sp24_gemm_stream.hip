// Small-m ("decode") GEMM kernels with an LDS ring: Y[m, n] = sum_k X[m, k] W[n, k].
//
// At decode sizes the product streams the weight once from HBM and is bound
// by that stream; X (at most a few hundred KB) is re-read from L2 by every
// workgroup.  These kernels give each workgroup one contiguous range of W
// rows (sized by the host so that the grid covers every CU with equal shares,
// e.g. 56 rows on each of 256 CUs for n = 14336; a multiple of 4 rows) and walk K in steps.  Every
// operand of a step -- the rows' compressed values and metadata words and the
// X rows -- goes from global memory straight into one buffer of an LDS ring
// with global_load_lds, in whole 64..256-byte row segments, STAGES-1 steps
// ahead of the step being multiplied; the X rows of a step are then read from
// LDS by every wave that needs them.
//
// Waves.  A workgroup has RBW x MW x KW waves: wave (rg, mg, kg) multiplies
// RB row blocks (16 W rows each, rows [16*RB*rg, 16*RB*(rg+1))) by MB token
// blocks (16 X rows each, token blocks [MB*mg, MB*(mg+1))) over units
// [kg*U, (kg+1)*U) of every step (a unit is 128 values of K; a step holds
// U*KW units).  A wave reads each X fragment once for its RB row blocks and
// each W fragment once for its MB token blocks; the MW waves along the tokens
// let one workgroup cover a few hundred tokens, so that W is streamed once.
// The KW partial tiles of a row block are summed through LDS in a fixed order
// at the end, and K slices of the grid (grid.z) through the split-K
// workspace, so results are bitwise reproducible.
//
// Instruction mapping (16 x 16 tiles; measured on gfx950 with one-hot
// probes).  The compressed operand is A, so W is A and X is B and the
// accumulator is a tile of Y^T: lane l, register i <-> W row 4*(l/16) + i,
// token l % 16.  Within a unit, A lane group q = l/16 holds the 32 K values
// [32q, 32q + 32) of its row (16 bytes of fp8 values and one metadata word);
// the sparse B operand holds two runs of K (the measured split-half layout),
// which for fp8 are the unit's bytes [64h + 16q, +16), h = 0, 1.  The bf16
// and dense variants use the same unit with their own instruction shapes.
// INT8 takes the integer forms of the fp8 instructions with the same operand
// layouts; its int32 accumulators become fp32 once, after the K loop.
//
// LDS rows are XOR-swizzled in 16-byte pieces so that the 16 rows read by one
// instruction fall on distinct bank groups; the LDS-DMA load writes lane i's
// bytes to slot i, so the swizzle is applied on the global side.
#include <atomic>

#include "sp24_common.hpp"
#include "sp24_dma.hpp"
#include "sp24_fp8.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kLdsBytes = kStreamLdsBytes;
// Quantising kernels (QX): a workgroup holds up to this many values of X in
// registers from the maximum to the cast (8-value vectors, spread over its
// threads: 4 per thread with 512 threads, 8 with 256; one token over K = 14336),
// so that X is read once; larger X is read twice, four loads at a time.  More
// per thread would cost the two-workgroup configurations their occupancy
// (128 VGPRs).
constexpr int kQxRegValues = 16384;
template <class C>
constexpr int qx_reg_vecs() {
  return kQxRegValues / 8 / C::NT > 0 ? kQxRegValues / 8 / C::NT : 1;
}

// BUDGET: LDS bytes the ring may take (less than the LDS when the kernel keeps a
// table of group scales beside it).
template <int DT, bool SPARSE, int RBW, int RB, int MW, int KW, int MB, int U, int SMAX,
          int BUDGET = kStreamLdsBytes>
struct StreamCfg {
  static constexpr int DT_ = DT, RBW_ = RBW, RB_ = RB, MW_ = MW, KW_ = KW, MB_ = MB, U_ = U;
  static constexpr bool SPARSE_ = SPARSE;
  static constexpr bool B8 = DT != SP24_BF16;  // one-byte codes (E4M3 or INT8)
  static constexpr bool I8 = DT == SP24_INT8;
  static constexpr int ESZ = B8 ? 1 : 2;
  static constexpr int NW = RBW * MW * KW, NT = NW * 64;
  static constexpr int BN = RBW * RB * 16, BM = MW * MB * 16;  // W rows, X rows per workgroup
  static constexpr int UPS = U * KW;                      // units of 128 K per step
  static constexpr int XU = 128 * ESZ;                    // X bytes per row per unit
  static constexpr int WU = (SPARSE ? 64 : 128) * ESZ;    // W bytes per row per unit
  static constexpr int MU = SPARSE ? 4 : 0;               // metadata words per row per unit
  static constexpr int XB = UPS * XU, WB = UPS * WU, MWD = UPS * MU;  // per row per step
  static constexpr int PX = XB / 16, PW = WB / 16;        // 16-byte pieces per row per step
  static constexpr int PXU = XU / 16, PWU = WU / 16;      // ... per unit
  static constexpr int W_OFF = 0, M_OFF = BN * WB, X_OFF = M_OFF + BN * MWD * 4;
  static constexpr int STAGE = X_OFF + BM * XB;           // bytes per LDS buffer
  static constexpr int STAGES = stream_stages(DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX, BUDGET);
  static constexpr bool FITS = stream_fits(DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX, BUDGET);
  // 16-byte operand pieces per lane per unit: A (per row block), B (per token block)
  static constexpr int AP = SPARSE ? (B8 ? 1 : 2) : (B8 ? 2 : 4);
  static constexpr int BP = B8 ? 2 : 4;
  // load instructions per step: 1 KB (dwordx4) for values and X, 256 B (dword) for metadata
  static constexpr int W_TOT = BN * WB / 1024, M_TOT = BN * MWD / 64, X_TOT = BM * XB / 1024;
  static constexpr int W_PER = (W_TOT + NW - 1) / NW, M_PER = (M_TOT + NW - 1) / NW,
                       X_PER = (X_TOT + NW - 1) / NW;
  // every wave issues at least this many loads per step
  static constexpr int MIN_PER_STEP = W_TOT / NW + M_TOT / NW + X_TOT / NW;
  static constexpr int RED = KW > 1 ? KW * RBW * MW * RB * MB * 1024 : 0;  // epilogue LDS bytes
  static constexpr int LDS = STAGES * STAGE > RED ? STAGES * STAGE : RED;
  static_assert(STAGE == stream_stage_bytes(DT, SPARSE, RBW, RB, MW, KW, MB, U), "one stage formula");
  static_assert(!FITS || (STAGES >= 2 && LDS <= kLdsBytes && STAGES * STAGE <= BUDGET), "LDS budget");
  static_assert(W_TOT * 1024 == BN * WB && X_TOT * 1024 == BM * XB && M_TOT * 64 == BN * MWD,
                "whole load instructions");
  static_assert(!FITS || MIN_PER_STEP * (STAGES - 2) < 64, "vmcnt range");
  static_assert(LDS == stream_ring_bytes(DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX, false, BUDGET),
                "one LDS formula");
  // X quantised by the kernel (QX): ring buffers without X rows, the X rows of
  // the workgroup's tokens and K slice after RING_QX
  static constexpr int STAGE_QX = X_OFF;
  static constexpr int RING_QX = stream_ring_bytes(DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX, true);
  static constexpr int MIN_PER_STEP_QX = W_TOT / NW + M_TOT / NW;
};

// s_waitcnt vmcnt(n) for a wave-uniform n in [LO, HI].
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vm_range<LO, MID>(n);
    else wait_vm_range<MID + 1, HI>(n);
  }
}

// Workgroup barrier for LDS data only: this wave's LDS accesses are done
// (lgkmcnt 0), then a bare s_barrier; vector-memory loads in flight (the ring's
// LDS-DMA loads) stay in flight, where __syncthreads() would wait for them.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Metadata words (MW per row): the 16 rows x 4 words of one read land on 64
// distinct banks.
template <int MW>
__device__ __forceinline__ int swzm(int r, int w) {
  if constexpr (MW <= 4) return w;
  else return w ^ (4 * ((r / (64 / MW)) & (MW / 4 - 1)));
}

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Per-lane sources of this wave's loads.  Load g of a stream (g = j*NW +
// wave) fills slots [64g, 64g + 64) of the stream's LDS region; step ks adds
// ks * UPS units to every source.
template <class C, bool QX>
struct StreamLoader {
  const uint8_t* wp[C::W_PER];
  const uint32_t* mp[C::M_PER > 0 ? C::M_PER : 1];
  const uint8_t* xp[C::X_PER];
  int wave;
  size_t mstep;  // metadata words of UPS 128-K blocks of all N rows

  __device__ __forceinline__ StreamLoader(const uint8_t* __restrict__ w,
                                          const uint32_t* __restrict__ meta,
                                          const uint8_t* __restrict__ x, int n0, int n_last,
                                          int m0, int M, int N, int K, int u0, int wave_, int lane)
      : wave(wave_), mstep((size_t)C::UPS * N * 4) {
    const size_t wrow = (size_t)(K / 128) * C::WU;
#pragma unroll
    for (int j = 0; j < C::W_PER; ++j) {
      const int p = (j * C::NW + wave) * 64 + lane, row = p / C::PW;
      const int sp = swz16<C::PW>(row, p % C::PW);
      const int n = min(n0 + row, n_last);  // rows past the range: clamp the load, never stored
      wp[j] = w + (size_t)n * wrow + (size_t)(u0 + sp / C::PWU) * C::WU + 16 * (sp % C::PWU);
    }
    if constexpr (C::SPARSE_) {
#pragma unroll
      for (int j = 0; j < C::M_PER; ++j) {
        const int p = (j * C::NW + wave) * 64 + lane, row = p / C::MWD;
        const int sw = swzm<C::MWD>(row, p % C::MWD);
        const int n = min(n0 + row, n_last);
        // unit u is metadata block u: every row's 4 words, row after row
        mp[j] = meta + (size_t)(u0 + sw / 4) * N * 4 + (size_t)n * 4 + (sw % 4);
      }
    }
    const size_t xrow = (size_t)K * C::ESZ;
#pragma unroll
    for (int j = 0; j < (QX ? 0 : C::X_PER); ++j) {
      const int p = (j * C::NW + wave) * 64 + lane, row = p / C::PX;
      const int sp = swz16<C::PX>(row, p % C::PX);
      const int m = min(m0 + row, M - 1);  // rows past M: clamp the load, never stored
      xp[j] = x + (size_t)m * xrow + (size_t)(u0 + sp / C::PXU) * C::XU + 16 * (sp % C::PXU);
    }
  }

  __device__ __forceinline__ void issue(uint8_t* buf, int ks) const {
#pragma unroll
    for (int j = 0; j < C::W_PER; ++j) {
      const int g = j * C::NW + wave;
      if (C::W_TOT % C::NW == 0 || g < C::W_TOT)
        dma16_nt(wp[j] + (size_t)ks * C::WB, buf + C::W_OFF + g * 1024);
    }
#pragma unroll
    for (int j = 0; j < C::M_PER; ++j) {
      const int g = j * C::NW + wave;
      if (C::M_TOT % C::NW == 0 || g < C::M_TOT)
        dma4_nt(mp[j] + (size_t)ks * mstep, buf + C::M_OFF + g * 256);
    }
#pragma unroll
    for (int j = 0; j < (QX ? 0 : C::X_PER); ++j) {
      const int g = j * C::NW + wave;
      if (C::X_TOT % C::NW == 0 || g < C::X_TOT)
        dma16(xp[j] + (size_t)ks * C::XB, buf + C::X_OFF + g * 1024);
    }
  }
};

__device__ __forceinline__ i32x4 lds16(const uint8_t* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// 16-byte piece (within its 128-K unit) that B operand piece e of lane group q
// takes from a token's row: sparse one-byte codes, run e: bytes [64e + 16q, +16);
// sparse bf16, instruction h = e >> 1, run hb = e & 1: K 64hb + 32(q>>1) + 16h +
// 8(q&1); dense one-byte codes: bytes [32q + 16e, +16); dense bf16: K [32e + 8q, +8).
template <class C>
__device__ __forceinline__ int b_piece(int e, int q) {
  if constexpr (C::SPARSE_ && C::B8) return 4 * e + q;
  else if constexpr (C::SPARSE_) return 8 * (e & 1) + 4 * (q >> 1) + 2 * (e >> 1) + (q & 1);
  else if constexpr (C::B8) return 2 * q + e;
  else return 4 * e + q;
}

// Operands of units kg*U .. kg*U + U - 1 of one step from LDS: A (W) and index
// words for the RB row blocks of row group rg, from the step's ring buffer; B
// (X) for the MB token blocks of token group mg, from X rows at xs + min(r,
// xlast) * xstride (a ring buffer: xs = buf + X_OFF, xstride = XB; resident X:
// the step's part of each row).
template <class C>
struct StreamOperands {
  i32x4 a[C::U_][C::RB_][C::AP];
  uint32_t ix[C::U_][C::RB_];
  i32x4 b[C::U_][C::MB_][C::BP];

  __device__ __forceinline__ void read(const uint8_t* __restrict__ buf, const uint8_t* __restrict__ xs,
                                       int xstride, int xlast, int rg, int mg, int kg, int lane) {
    constexpr int MB = C::MB_, U = C::U_, RB = C::RB_;
    constexpr bool B8 = C::B8, SPARSE = C::SPARSE_;
    const int q = lane >> 4, r = lane & 15;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = kg * U + u;  // unit within the step
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int wrow = 16 * (RB * rg + rb) + r;
        const uint8_t* wr = buf + C::W_OFF + wrow * C::WB;
#pragma unroll
        for (int e = 0; e < C::AP; ++e) {
          int c;
          if constexpr (SPARSE && B8) c = v * C::PWU + q;                  // K [32q, +32)
          else if constexpr (SPARSE) c = v * C::PWU + 2 * q + e;           // e-th 16 K of [32q, +32)
          else if constexpr (B8) c = v * C::PWU + 2 * q + e;               // K [32q, +32)
          else c = v * C::PWU + 4 * e + q;                                 // K [32e + 8q, +8)
          a[u][rb][e] = lds16(wr + 16 * swz16<C::PW>(wrow, c));
        }
        if constexpr (SPARSE)
          ix[u][rb] = *reinterpret_cast<const uint32_t*>(buf + C::M_OFF + wrow * C::MWD * 4 +
                                                         4 * swzm<C::MWD>(wrow, 4 * v + q));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int xrow = min(16 * (MB * mg + mb) + r, xlast);
        const uint8_t* xr = xs + xrow * xstride;
#pragma unroll
        for (int e = 0; e < C::BP; ++e)
          b[u][mb][e] = lds16(xr + 16 * swz16<C::PX>(xrow, v * C::PXU + b_piece<C>(e, q)));
      }
    }
  }
};

// The matrix instruction(s) of unit u for row block rb and token block mb: c += W x X.
template <class C>
__device__ __forceinline__ void stream_mfma_one(f32x4& c, const StreamOperands<C>& o, int u, int rb, int mb) {
  constexpr bool B8 = C::B8, I8 = C::I8, SPARSE = C::SPARSE_;
  if constexpr (SPARSE && I8) {
    c = __builtin_bit_cast(f32x4, __builtin_amdgcn_smfmac_i32_16x16x128_i8(
                                      o.a[u][rb][0], cat8(o.b[u][mb][0], o.b[u][mb][1]),
                                      __builtin_bit_cast(i32x4, c), (int)o.ix[u][rb], 0, 0));
  } else if constexpr (SPARSE && B8) {
    c = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(o.a[u][rb][0], cat8(o.b[u][mb][0], o.b[u][mb][1]), c,
                                                      (int)o.ix[u][rb], 0, 0);
  } else if constexpr (SPARSE) {
    c = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
        __builtin_bit_cast(bf16x8, o.a[u][rb][0]), __builtin_bit_cast(bf16x16, cat8(o.b[u][mb][0], o.b[u][mb][1])),
        c, (int)o.ix[u][rb], 0, 0);
    c = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
        __builtin_bit_cast(bf16x8, o.a[u][rb][1]), __builtin_bit_cast(bf16x16, cat8(o.b[u][mb][2], o.b[u][mb][3])),
        c, (int)o.ix[u][rb], 0, 1);
  } else if constexpr (I8) {
    // dense INT8: two instructions of K=64 over the lane group's 32 bytes
#pragma unroll
    for (int e = 0; e < 2; ++e)
      c = __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[u][rb][e], o.b[u][mb][e],
                                                                          __builtin_bit_cast(i32x4, c), 0, 0, 0));
  } else if constexpr (B8) {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat8(o.a[u][rb][0], o.a[u][rb][1]),
                                                         cat8(o.b[u][mb][0], o.b[u][mb][1]), c, 0, 0, 0, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.a[u][rb][e]),
                                                  __builtin_bit_cast(bf16x8, o.b[u][mb][e]), c, 0, 0, 0);
  }
}

// Units kg*U .. kg*U + U - 1 of one step for the RB row blocks of row group
// rg and the MB token blocks of token group mg.  All LDS reads of the step
// are issued before its matrix instructions.
template <class C>
__device__ __forceinline__ void stream_mma(f32x4 (&acc)[C::RB_][C::MB_], const uint8_t* __restrict__ buf,
                                           const uint8_t* __restrict__ xs, int xstride, int xlast,
                                           int rg, int mg, int kg, int lane) {
  StreamOperands<C> o;
  o.read(buf, xs, xstride, xlast, rg, mg, kg, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < C::U_; ++u)
#pragma unroll
    for (int rb = 0; rb < C::RB_; ++rb)
#pragma unroll
      for (int mb = 0; mb < C::MB_; ++mb) stream_mfma_one<C>(acc[rb][mb], o, u, rb, mb);
}

// Group scales (sparse FP8): the products of every unit of a step go to fresh
// tiles t; each tile is added to the accumulator times fp32(sx * sw) of its
// unit's group (sw of the lane's four W rows from tw, [group][row] over the
// workgroup's rows; sx of its token from tx, [group][token]).
template <class C>
struct GsTiles {
  f32x4 t[C::U_][C::RB_][C::MB_];
  f32x4 s[C::U_][C::RB_][C::MB_];  // the scale of each element of t

  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int u = 0; u < C::U_; ++u)
#pragma unroll
      for (int rb = 0; rb < C::RB_; ++rb)
#pragma unroll
        for (int mb = 0; mb < C::MB_; ++mb) t[u][rb][mb] = s[u][rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // acc += t * s, unit by unit in order
  __device__ __forceinline__ void fold(f32x4 (&acc)[C::RB_][C::MB_]) const {
#pragma unroll
    for (int u = 0; u < C::U_; ++u)
#pragma unroll
      for (int rb = 0; rb < C::RB_; ++rb)
#pragma unroll
        for (int mb = 0; mb < C::MB_; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][mb][i] += t[u][rb][mb][i] * s[u][rb][mb][i];
  }
};

// One step with group scales: the step's products into `cur` (with their scales),
// then the previous step's tiles `prev` folded into the accumulator while the
// matrix instructions run.  `unit0` is the step's first unit within the K slice.
template <class C>
__device__ __forceinline__ void stream_gs_step(GsTiles<C>& cur, const GsTiles<C>& prev, f32x4 (&acc)[C::RB_][C::MB_],
                                               const uint8_t* __restrict__ buf, int rg, int mg, int kg, int lane,
                                               const float* __restrict__ tw, const float* __restrict__ tx, int unit0,
                                               int group_units) {
  static_assert(C::SPARSE_ && C::DT_ == SP24_FP8_E4M3, "group scales: sparse FP8");
  StreamOperands<C> o;
  o.read(buf, buf + C::X_OFF, C::XB, C::BM - 1, rg, mg, kg, lane);
  const int q = lane >> 4, r = lane & 15;
  f32x4 sw[C::U_][C::RB_];
  float sx[C::U_][C::MB_];
#pragma unroll
  for (int u = 0; u < C::U_; ++u) {
    const int g = (unit0 + kg * C::U_ + u) / group_units;
#pragma unroll
    for (int rb = 0; rb < C::RB_; ++rb)
      sw[u][rb] = *reinterpret_cast<const f32x4*>(tw + g * C::BN + 16 * (C::RB_ * rg + rb) + 4 * q);
#pragma unroll
    for (int mb = 0; mb < C::MB_; ++mb) sx[u][mb] = tx[g * C::BM + 16 * (C::MB_ * mg + mb) + r];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < C::U_; ++u)
#pragma unroll
    for (int rb = 0; rb < C::RB_; ++rb)
#pragma unroll
      for (int mb = 0; mb < C::MB_; ++mb) {
        cur.t[u][rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        stream_mfma_one<C>(cur.t[u][rb][mb], o, u, rb, mb);
      }
  prev.fold(acc);
#pragma unroll
  for (int u = 0; u < C::U_; ++u)
#pragma unroll
    for (int rb = 0; rb < C::RB_; ++rb)
#pragma unroll
      for (int mb = 0; mb < C::MB_; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cur.s[u][rb][mb][i] = sx[u][mb] * sw[u][rb][i];
}

// QX: X is bf16 (xh) and quantised here, exactly as the quantisers do it (same
// key, scale and cast).  Per tensor (QROWS false): the scale of the whole of
// X; block (0, 0, 0) stores it to sx_out.  Per token (QROWS): each workgroup
// reads only its own tokens, row r gets the scale of its own maximum, and the
// blocks with blockIdx.x = blockIdx.z = 0 store their rows' scales to
// sx_out[m].  X rows hold xk values; with lift = N (3..8) they are lifted to the
// SlideSparse windows on the way into LDS (the GEMM's K is then K' = xk (2N-2)/N),
// with lift = 0 they are taken as they are (xk = K).
//
// GS (group scales, sparse FP8, X codes given): X row m and W row n carry one
// scale per group of group_units units of 128 K (x_gscale [M, n_groups],
// w_gscale [N, n_groups]).  The scales of the workgroup's rows and tokens for its
// K slice are loaded once into an LDS table beside the ring; every unit's
// products are added to the accumulator times fp32(sx * sw) of its group, so the
// epilogue applies no scale.  Otherwise W row n's scale is w_scale[n * ws_step].
template <class C, bool PARTIAL, bool QX, bool QROWS = false, bool GS = false>
__global__ __launch_bounds__(C::NT) void gemm_stream_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const uint32_t* __restrict__ meta,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, uint16_t* __restrict__ y,
    float* __restrict__ partial, int M, int N, int K, int rows_per_wg, int units_per_slice,
    const uint16_t* __restrict__ xh, float* __restrict__ sx_out, int xs_step, int xk, int lift, int ws_step,
    const float* __restrict__ x_gscale, const float* __restrict__ w_gscale, int group_units, int n_groups,
    int x_stage) {
  static_assert(!(GS && QX), "group scales take X codes");
  constexpr int MB = C::MB_, RB = C::RB_, RBW = C::RBW_, KW = C::KW_, STAGES = C::STAGES;
  constexpr int STAGE = QX ? C::STAGE_QX : C::STAGE;
  // QX: the X codes sit in an array of their own (dynamic LDS, sized by the
  // host: the workgroup's rows times the row stride), so the compiler can tell
  // its reads from the LDS-DMA writes into the ring (it would otherwise wait for
  // every load in flight before each step's reads).  The ring array holds the
  // ring without X rows and the reduction of the KW partial tiles
  // (stream_ring_bytes with qx); it is never smaller than that.
  constexpr int LDS_QX = C::RING_QX;
  __shared__ __attribute__((aligned(16))) uint8_t lds[QX ? LDS_QX : C::LDS];
  // per tensor: each wave's largest key; per token: each row's largest key
  __shared__ uint32_t wave_max[QX ? (QROWS ? C::BM : C::NW) : 1];
  // per token: each row's scale and the reciprocal of its divisor (QDiv)
  __shared__ float row_sr[QX && QROWS ? 2 * C::BM : 1];
  // dynamic LDS, sized by the host: QX, the X codes; GS, the group scales of this
  // workgroup's rows ([group][row]) and tokens ([group][token]) for the K slice (at
  // most kStreamGsBytes)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  float* const gstab = reinterpret_cast<float*>(dyn_lds);
  // QX per tensor with x_stage > 0: all of X (bf16, x_stage = 2 M K bytes) is staged
  // in dyn_lds[0, x_stage) and the codes follow it
  if constexpr (!QX || QROWS) x_stage = 0;
  uint8_t* const xcodes = dyn_lds + x_stage;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar
  const int rg = wave % RBW, mg = (wave / RBW) % C::MW_, kg = wave / (RBW * C::MW_);
  const int n0 = blockIdx.x * rows_per_wg, m0 = blockIdx.y * C::BM;
  const int n_end = min(N, n0 + rows_per_wg);
  const int u0 = blockIdx.z * units_per_slice;
  const int nks = units_per_slice / C::UPS;  // the host keeps units_per_slice a multiple of UPS

  f32x4 acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of STAGES buffers.  At the top of step ks a wave waits for its own
  // loads of step ks; the barrier then makes every wave's loads visible and
  // guarantees that every wave has finished reading buffer (ks - 1) % STAGES,
  // which receives the loads of step ks + STAGES - 1 while step ks is
  // multiplied.  A bare s_barrier: __syncthreads() adds a release fence that
  // waits for every outstanding LDS-DMA load and would drain the ring.
  const StreamLoader<C, QX> ld(w, meta, x, n0, n_end - 1, m0, M, N, K, u0, wave, lane);

  // QX: take the scale from all of X and cast this workgroup's tokens over its
  // K slice into LDS (the dynamic array), piece p of a step's part of
  // row r in slot swz16(r, p) as a ring buffer would hold it.
  // QX: the ring's first loads (W and metadata only) go out before the
  // prologue, so they travel while X is read.  Loads complete in issue order,
  // so X loaded into registers after them is usable only once they have
  // landed, and the prologue's __syncthreads() waits for every load in
  // flight: the first steps of W arrive before the prologue ends and the ring
  // refills from empty after it.  With x_stage (per tensor, X small enough and
  // the LDS to hold it without losing a workgroup per CU) X goes into LDS by
  // LDS-DMA before the ring's loads: the wave waits for its own X loads only
  // (the ring's loads, issued after them, may stay in flight), and the
  // prologue's barriers wait for LDS accesses only, so W streams on while X is
  // reduced and cast.
  if constexpr (QX && QROWS) {  // the rows' maxima start at 0 (before any load is in flight)
    if (threadIdx.x < C::BM) wave_max[threadIdx.x] = 0u;
    __syncthreads();
  }
  int ring_prologue_loads = 0;  // this wave's ring loads issued after its X staging loads
  if constexpr (QX && !QROWS) {
    if (x_stage > 0) {
      const int nvec = M * K / 8, ninstr = (nvec + 63) / 64;  // M K <= kQxRegValues (host)
      for (int g = wave; g < ninstr; g += C::NW) {
        const int i = g * 64 + lane;
        if (i < nvec) dma16(xh + (size_t)i * 8, dyn_lds + g * 1024);
      }
      int per = 0;
#pragma unroll
      for (int j = 0; j < C::W_PER; ++j) per += (j * C::NW + wave < C::W_TOT) ? 1 : 0;
#pragma unroll
      for (int j = 0; j < C::M_PER; ++j) per += (j * C::NW + wave < C::M_TOT) ? 1 : 0;
      ring_prologue_loads = per * min(STAGES - 1, nks);
    }
  }
  if constexpr (QX) {
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < nks) ld.issue(lds + p * STAGE, p);
  }
  float sx = 1.0f;
  uint8_t* const xres = xcodes;
  const int mrows = min(C::BM, M - m0);
  const int xrs = (int)stream_qx_row_bytes((int64_t)units_per_slice * 128, C::XB);
  // the LDS slot of the code at K offset kk (within the slice) of token row rr
  auto slot = [&](int rr, int kk) {
    const int st = kk / C::XB, within = kk - st * C::XB;
    return xres + rr * xrs + st * C::XB + 16 * swz16<C::PX>(rr, within / 16) + (within & 15);
  };
  if constexpr (QX && QROWS) {
    const int tid = threadIdx.x;
    const int vpr = xk / 8;                    // 8-value vectors per X row (xk % 8 == 0)
    const int nv = mrows * vpr;                // this workgroup's tokens only
    const u32x4* xv = reinterpret_cast<const u32x4*>(xh + (size_t)m0 * xk);
    uint32_t* row_key = wave_max;
    constexpr int RV = qx_reg_vecs<C>();
    const bool in_regs = nv <= RV * C::NT;
    u32x4 xr[RV];
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const int i = tid + r * C::NT;
        xr[r] = i < nv ? xv[i] : u32x4{0u, 0u, 0u, 0u};
        if (i < nv) atomicMax(&row_key[i / vpr], key_max8(xr[r]));
      }
    } else {
      int i = tid;
      for (; i + 3 * C::NT < nv; i += 4 * C::NT) {  // four loads in flight
        const u32x4 a = xv[i], b = xv[i + C::NT], c = xv[i + 2 * C::NT], d = xv[i + 3 * C::NT];
        atomicMax(&row_key[i / vpr], key_max8(a));
        atomicMax(&row_key[(i + C::NT) / vpr], key_max8(b));
        atomicMax(&row_key[(i + 2 * C::NT) / vpr], key_max8(c));
        atomicMax(&row_key[(i + 3 * C::NT) / vpr], key_max8(d));
      }
      for (; i < nv; i += C::NT) atomicMax(&row_key[i / vpr], key_max8(xv[i]));
    }
    __syncthreads();
    if (tid < mrows) {
      const QDiv d = qdiv<SP24_FP8_E4M3>(row_key[tid]);
      row_sr[2 * tid] = d.s;
      row_sr[2 * tid + 1] = d.r;
      if (sx_out != nullptr && blockIdx.x == 0 && blockIdx.z == 0) sx_out[m0 + tid] = d.s;
    }
    __syncthreads();
    const int k0 = u0 * 128, kslice = units_per_slice * 128;
    // vector i: 8 codes at K offset kk of row rr, or (lifted) its 4 code pairs: pair
    // P = kk/2 + t is pair j = P % N of block b = P / N, which window j (j <= N-2)
    // takes at its positions 0, 1 and window j - 1 (j >= 1) at its positions 2, 3
    auto cast_vec = [&](int i, u32x4 d) {
      const int rr = i / vpr, kk = (i - rr * vpr) * 8;
      const u32x2 c8 = cast8(d, qdiv_from(row_sr[2 * rr], row_sr[2 * rr + 1]));
      if (lift == 0) {
        const int kp = kk - k0;
        if (kp >= 0 && kp < kslice) *reinterpret_cast<u32x2*>(slot(rr, kp)) = c8;
        return;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t c2 = (uint16_t)(c8[t >> 1] >> (16 * (t & 1)));
        const int pr = kk / 2 + t, b = pr / lift, j = pr - b * lift;
        const int base = b * 4 * (lift - 1) - k0;
        int kp = base + 4 * j;
        if (j <= lift - 2 && kp >= 0 && kp < kslice) *reinterpret_cast<uint16_t*>(slot(rr, kp)) = c2;
        kp = base + 4 * (j - 1) + 2;
        if (j >= 1 && kp >= 0 && kp < kslice) *reinterpret_cast<uint16_t*>(slot(rr, kp)) = c2;
      }
    };
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < RV; ++r)
        if (tid + r * C::NT < nv) cast_vec(tid + r * C::NT, xr[r]);
    } else {
      int i = tid;
      for (; i + 3 * C::NT < nv; i += 4 * C::NT) {  // four loads in flight
        const u32x4 a = xv[i], b = xv[i + C::NT], c = xv[i + 2 * C::NT], d = xv[i + 3 * C::NT];
        cast_vec(i, a);
        cast_vec(i + C::NT, b);
        cast_vec(i + 2 * C::NT, c);
        cast_vec(i + 3 * C::NT, d);
      }
      for (; i < nv; i += C::NT) cast_vec(i, xv[i]);
    }
    __syncthreads();  // the codes are in LDS for every wave
  } else if constexpr (QX) {
    const int tid = threadIdx.x;
    const u32x4* xv = reinterpret_cast<const u32x4*>(xh);
    const int64_t nvec = (int64_t)M * K / 8;  // 8-value vectors of X (K % 8 == 0: none spans two rows)
    const int kslice = units_per_slice * 128;
    // small X (every decode token at once): each thread keeps its vectors in
    // registers from the maximum to the cast, one pass over global memory
    constexpr int RV = qx_reg_vecs<C>();
    const bool in_regs = nvec <= (int64_t)RV * C::NT;
    u32x4 xr[RV];
    uint32_t mk = 0;
    if (x_stage > 0) {  // in_regs holds (the host stages only X of at most kQxRegValues values)
      // this wave's staging loads have landed (more than 63 ring loads after them:
      // waiting for 63 still implies them); the barrier makes every wave's visible
      wait_vm_range<0, 63>(min(ring_prologue_loads, 63));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const int i = tid + r * C::NT;
        xr[r] = i < (int)nvec ? *reinterpret_cast<const u32x4*>(dyn_lds + (size_t)i * 16) : u32x4{0u, 0u, 0u, 0u};
        mk = max(mk, key_max8(xr[r]));
      }
    } else if (in_regs) {  // nvec <= RV * NT: 32-bit indices
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const int i = tid + r * C::NT;
        xr[r] = i < (int)nvec ? xv[i] : u32x4{0u, 0u, 0u, 0u};
        mk = max(mk, key_max8(xr[r]));
      }
    } else {
      int64_t i = tid;
      for (; i + 3 * C::NT < nvec; i += 4 * C::NT) {  // four loads in flight
        const u32x4 a = xv[i], b = xv[i + C::NT], c = xv[i + 2 * C::NT], d = xv[i + 3 * C::NT];
        mk = max(mk, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
      }
      for (; i < nvec; i += C::NT) mk = max(mk, key_max8(xv[i]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, off, 64));
    if (lane == 0) wave_max[wave] = mk;
    if (x_stage > 0) lds_barrier();
    else __syncthreads();
#pragma unroll
    for (int g = 0; g < C::NW; ++g) mk = max(mk, wave_max[g]);
    const QDiv sxd = qdiv<SP24_FP8_E4M3>(mk);
    sx = sxd.s;
    if (sx_out != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) *sx_out = sx;
    // codes of value kk (relative to the K slice) of token row rr
    auto put = [&](int rr, int kk, u32x2 c8) { *reinterpret_cast<u32x2*>(slot(rr, kk)) = c8; };
    const int k0 = u0 * 128;
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const int i = tid + r * C::NT;
        if (i >= (int)nvec) continue;
        const int row = 8 * i / K, kk = 8 * i - row * K - k0;
        if (row >= m0 && row < m0 + mrows && kk >= 0 && kk < kslice) put(row - m0, kk, cast8(xr[r], sxd));
      }
    } else {
      const int vpr = kslice / 8;  // 8-value vectors per row of the slice
      const uint16_t* xs0 = xh + (size_t)m0 * K + k0;
      auto src = [&](int v) {
        const int rr = v / vpr;
        return reinterpret_cast<const u32x4*>(xs0 + (size_t)rr * K + (v - rr * vpr) * 8);
      };
      auto put_vec = [&](int v, u32x4 d) {
        const int rr = v / vpr;
        put(rr, (v - rr * vpr) * 8, cast8(d, sxd));
      };
      const int nv = mrows * vpr;
      int v = tid;
      for (; v + 3 * C::NT < nv; v += 4 * C::NT) {  // four loads in flight
        const u32x4 a = *src(v), b = *src(v + C::NT), c = *src(v + 2 * C::NT), d = *src(v + 3 * C::NT);
        put_vec(v, a);
        put_vec(v + C::NT, b);
        put_vec(v + 2 * C::NT, c);
        put_vec(v + 3 * C::NT, d);
      }
      for (; v < nv; v += C::NT) put_vec(v, *src(v));
    }
    if (x_stage > 0) lds_barrier();  // the codes are in LDS for every wave
    else __syncthreads();
  }

  if constexpr (GS) {
    // the group scales of the K slice, before any ring load is in flight (the host
    // keeps slices whole groups and the table within kStreamGsBytes)
    const int gslice = units_per_slice / group_units, g0 = u0 / group_units;
    for (int e = threadIdx.x; e < gslice * C::BN; e += C::NT) {
      const int g = e / C::BN, row = e - g * C::BN;
      gstab[e] = w_gscale[(size_t)min(n0 + row, n_end - 1) * n_groups + g0 + g];
    }
    float* tx = gstab + gslice * C::BN;
    for (int e = threadIdx.x; e < gslice * C::BM; e += C::NT) {
      const int g = e / C::BM, tok = e - g * C::BM;
      tx[e] = x_gscale[(size_t)min(m0 + tok, M - 1) * n_groups + g0 + g];
    }
    __syncthreads();
  }
  if constexpr (!QX) {
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < nks) ld.issue(lds + p * STAGE, p);
  }
  // The top of step ks: this wave's loads of the step have landed and every wave
  // is done with the buffer the loads of step ks + STAGES - 1 go to; returns the
  // step's buffer.
  auto ring_step = [&](int ks) {
    wait_later<QX ? C::MIN_PER_STEP_QX : C::MIN_PER_STEP, STAGES - 2>(min(nks - 1 - ks, STAGES - 2));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // LDS reads stay after the barrier
    const int nxt = ks + STAGES - 1;
    if (nxt < nks) ld.issue(lds + (nxt % STAGES) * STAGE, nxt);
    return static_cast<const uint8_t*>(lds + (ks % STAGES) * STAGE);
  };
  if constexpr (GS) {
    // Each step's products go to fresh tiles, which are scaled and added one step
    // later, so that the matrix instructions of step ks + 1 run while the vector
    // unit folds step ks (two sets of tiles, the loop taken two steps at a time).
    const float* tx = gstab + (units_per_slice / group_units) * C::BN;
    GsTiles<C> t0, t1;
    t1.clear();
    int ks = 0;
    for (; ks + 1 < nks; ks += 2) {
      stream_gs_step<C>(t0, t1, acc, ring_step(ks), rg, mg, kg, lane, gstab, tx, ks * C::UPS, group_units);
      stream_gs_step<C>(t1, t0, acc, ring_step(ks + 1), rg, mg, kg, lane, gstab, tx, (ks + 1) * C::UPS,
                        group_units);
    }
    if (ks < nks) {
      stream_gs_step<C>(t0, t1, acc, ring_step(ks), rg, mg, kg, lane, gstab, tx, ks * C::UPS, group_units);
      t0.fold(acc);
    } else {
      t1.fold(acc);
    }
  } else {
    for (int ks = 0; ks < nks; ++ks) {
      const uint8_t* buf = ring_step(ks);
      if constexpr (QX)
        stream_mma<C>(acc, buf, xres + ks * C::XB, xrs, mrows - 1, rg, mg, kg, lane);
      else
        stream_mma<C>(acc, buf, buf + C::X_OFF, C::XB, C::BM - 1, rg, mg, kg, lane);
    }
  }

  if constexpr (C::I8)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][mb][i] = i32_bits_to_f32(acc[rb][mb][i]);

  // Sum the KW partial tiles of each row block in wave order kg = 0, 1, ...
  // Tile (rb, mb) of wave (rg, mg, kg) sits at
  // red[((((kg*MW + mg)*RBW + rg)*RB + rb)*MB + mb)*256 ...].
  if constexpr (KW > 1) {
    __syncthreads();  // every wave is done reading the ring
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(((((kg * C::MW_ + mg) * RBW + rg) * RB + rb) * MB + mb) * 4 + i) * 64 + lane] = acc[rb][mb][i];
    __syncthreads();
    if (kg != 0) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = red[((((mg * RBW + rg) * RB + rb) * MB + mb) * 4 + i) * 64 + lane];
#pragma unroll
          for (int g = 1; g < KW; ++g)
            s += red[(((((g * C::MW_ + mg) * RBW + rg) * RB + rb) * MB + mb) * 4 + i) * 64 + lane];
          acc[rb][mb][i] = s;
        }
  }

  const int q = lane >> 4, c = lane & 15;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = n0 + 16 * (RB * rg + rb) + 4 * q;  // accumulator registers 0..3: rows n .. n + 3
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + 16 * (MB * mg + mb) + c;
      if (m >= M || n >= n_end) continue;
      const f32x4 v = acc[rb][mb];
      if constexpr (PARTIAL) {
        float* pr = partial + ((size_t)blockIdx.z * M + m) * N;
        if (n + 3 < n_end && (N & 3) == 0) {
          *reinterpret_cast<f32x4*>(pr + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_end) pr[n + e] = v[e];
        }
      } else {
        uint16_t* yr = y + (size_t)m * N;
        // FP8, INT8: fp32(sx * sw) with the scales of X row m and W row n + e (one per
        // tensor: step 0); GS: the group scales are applied already
        float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (C::B8 && !GS) {
          float sxm;
          if constexpr (QX && QROWS) sxm = scale_from_key(wave_max[m - m0]);
          else sxm = QX ? sx : x_scale[(size_t)m * xs_step];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[e] = sxm * w_scale[(size_t)min(n + e, n_end - 1) * ws_step];
        }
        const uint32_t lo = f32_to_bf16_rne(v[0] * sc[0]) | (f32_to_bf16_rne(v[1] * sc[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(v[2] * sc[2]) | (f32_to_bf16_rne(v[3] * sc[3]) << 16);
        if (n + 3 < n_end && (N & 3) == 0) {
          *reinterpret_cast<u32x2*>(yr + n) = u32x2{lo, hi};
        } else {
          const uint32_t h[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_end) yr[n + e] = (uint16_t)h[e];
        }
      }
    }
  }
}

// Compute units of the current device (queried once per device; 256 if the query fails).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Rounds of workgroups a launch of `grid` workgroups of `lds` bytes each runs in,
// as far as the LDS decides how many a CU holds.
int64_t lds_rounds(int64_t grid, int64_t lds) {
  const int64_t per_cu = kStreamLdsBytes / (lds > 0 ? lds : 1);
  const int64_t at_once = (per_cu > 0 ? per_cu : 1) * device_cus();
  return (grid + at_once - 1) / at_once;
}

template <int DT, bool SPARSE, int RBW, int RB, int MW, int KW, int MB, int U, int SMAX>
hipError_t launch_stream_cfg(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  using C = StreamCfg<DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX>;
  if constexpr (!C::FITS) {
    return hipErrorInvalidConfiguration;  // the planner never picks it for this operand type
  } else {
    const dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(C::NT);
    const int units_per_slice = a.k / 128 / p.split_k;
    if (p.tile_n > C::BN || p.tile_m != C::BM || p.waves != C::NW || units_per_slice % C::UPS != 0)
      return hipErrorInvalidConfiguration;
    const uint8_t* x = static_cast<const uint8_t*>(a.x);
    const uint8_t* w = static_cast<const uint8_t*>(a.w);
    if (a.x_bf16 != nullptr) {
      if constexpr (DT == SP24_FP8_E4M3 && SPARSE && stream_qx_fits(RBW, RB, MW, KW, MB, U, SMAX, false)) {
        // the X rows of a workgroup (dynamic LDS) must fit what the ring leaves
        const int64_t rows = a.m < C::BM ? a.m : C::BM;
        const int64_t xbytes = rows * stream_qx_row_bytes((int64_t)units_per_slice * 128, C::XB);
        if (xbytes > stream_qx_room(RBW, RB, MW, KW, MB, U, SMAX, a.x_rows != 0))
          return hipErrorInvalidConfiguration;
        const size_t dyn = (size_t)xbytes;
        const int xk = a.x_lift ? a.k / (4 * (a.x_lift - 1)) * (2 * a.x_lift) : a.k;
        if (a.x_rows) {
          if constexpr (stream_qx_fits(RBW, RB, MW, KW, MB, U, SMAX, true)) {
            if (p.split_k > 1)
              hipLaunchKernelGGL((gemm_stream_kernel<C, true, true, true>), grid, block, dyn, s, x, w, a.meta,
                                 a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n,
                                 units_per_slice, a.x_bf16, a.x_scale_out, 0, xk, a.x_lift,
                             a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, 0);
            else
              hipLaunchKernelGGL((gemm_stream_kernel<C, false, true, true>), grid, block, dyn, s, x, w, a.meta,
                                 a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n,
                                 units_per_slice, a.x_bf16, a.x_scale_out, 0, xk, a.x_lift,
                             a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, 0);
          } else {
            return hipErrorInvalidConfiguration;
          }
        } else if (a.x_lift != 0) {
          return hipErrorInvalidValue;  // lifting is per token only
        } else {
          // stage X (bf16) in LDS ahead of the codes when it is small enough to stay in
          // registers from the maximum to the cast, fits what the ring leaves, and adds
          // no round of workgroups (the LDS per workgroup can lower how many a CU holds)
          const int64_t stage = 2 * (int64_t)a.m * a.k;
          const int64_t base = kStreamLdsBytes - stream_qx_room(RBW, RB, MW, KW, MB, U, SMAX, false) + xbytes;
          const int64_t grid_n = (int64_t)p.grid_x * p.grid_y * p.grid_z;
          const bool staged = (int64_t)a.m * a.k <= (int64_t)kQxRegValues &&
                              xbytes + stage <= stream_qx_room(RBW, RB, MW, KW, MB, U, SMAX, false) &&
                              lds_rounds(grid_n, base + stage) == lds_rounds(grid_n, base);
          const int xst = staged ? (int)stage : 0;
          const size_t dyn2 = dyn + (size_t)xst;
          if (p.split_k > 1)
            hipLaunchKernelGGL((gemm_stream_kernel<C, true, true>), grid, block, dyn2, s, x, w, a.meta, a.x_scale,
                               a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice, a.x_bf16,
                               a.x_scale_out, 0, a.k, 0,
                               a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, xst);
          else
            hipLaunchKernelGGL((gemm_stream_kernel<C, false, true>), grid, block, dyn2, s, x, w, a.meta, a.x_scale,
                               a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice, a.x_bf16,
                               a.x_scale_out, 0, a.k, 0,
                               a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, xst);
        }
        return hipGetLastError();
      } else {
        return hipErrorInvalidConfiguration;
      }
    }
    if (a.group_units > 0) {
      // group scales: the same configuration with its ring inside kStreamGsBudget
      if constexpr (DT == SP24_FP8_E4M3 && SPARSE && stream_gs_fits(RBW, RB, MW, KW, MB, U, SMAX)) {
        using CG = StreamCfg<DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX, kStreamGsBudget>;
        const int64_t gslice = units_per_slice / a.group_units;
        if (units_per_slice % a.group_units != 0 || gslice * (CG::BN + CG::BM) * 4 > kStreamGsBytes ||
            a.x_gscale == nullptr || a.w_gscale == nullptr)
          return hipErrorInvalidConfiguration;
        const size_t tab = (size_t)gslice * (CG::BN + CG::BM) * 4;  // dynamic LDS: the scale table
        if (p.split_k > 1)
          hipLaunchKernelGGL((gemm_stream_kernel<CG, true, false, false, true>), grid, block, tab, s, x, w, a.meta,
                             a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice,
                             (const uint16_t*)nullptr, (float*)nullptr, 0, a.k, 0, 0, a.x_gscale, a.w_gscale,
                             a.group_units, a.n_groups, 0);
        else
          hipLaunchKernelGGL((gemm_stream_kernel<CG, false, false, false, true>), grid, block, tab, s, x, w, a.meta,
                             a.x_scale, a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice,
                             (const uint16_t*)nullptr, (float*)nullptr, 0, a.k, 0, 0, a.x_gscale, a.w_gscale,
                             a.group_units, a.n_groups, 0);
        return hipGetLastError();
      } else {
        return hipErrorInvalidConfiguration;
      }
    }
    if (p.split_k > 1)
      hipLaunchKernelGGL((gemm_stream_kernel<C, true, false>), grid, block, 0, s, x, w, a.meta, a.x_scale,
                         a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice,
                         (const uint16_t*)nullptr, (float*)nullptr, a.x_scale_step, a.k, 0,
                             a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, 0);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<C, false, false>), grid, block, 0, s, x, w, a.meta, a.x_scale,
                         a.w_scale, a.y, a.partial, a.m, a.n, a.k, p.tile_n, units_per_slice,
                         (const uint16_t*)nullptr, (float*)nullptr, a.x_scale_step, a.k, 0,
                             a.w_scale_step, (const float*)nullptr, (const float*)nullptr, 0, 0, 0);
    return hipGetLastError();
  }
}

template <int DT, bool SPARSE>
hipError_t launch_stream_dt(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  switch (p.config - kStreamBase) {
#define SP24_STREAM_CASE(ID, RBW, RB, MW, KW, MB, U, SMAX) \
  case ID: return launch_stream_cfg<DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX>(a, p, s);
    SP24_STREAM_CONFIGS(SP24_STREAM_CASE)
#undef SP24_STREAM_CASE
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  if (a.dtype == SP24_FP8_E4M3)
    return a.sparse ? launch_stream_dt<SP24_FP8_E4M3, true>(a, p, s)
                    : launch_stream_dt<SP24_FP8_E4M3, false>(a, p, s);
  if (a.dtype == SP24_INT8)
    return a.sparse ? launch_stream_dt<SP24_INT8, true>(a, p, s) : launch_stream_dt<SP24_INT8, false>(a, p, s);
  return a.sparse ? launch_stream_dt<SP24_BF16, true>(a, p, s) : launch_stream_dt<SP24_BF16, false>(a, p, s);
}

}  // namespace sp24
