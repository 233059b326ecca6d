// Host-side launch functions of the libsp24 kernels.  Arguments are already
// validated by the C ABI layer (sp24_api.hip) when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sp24.h"

namespace sp24 {

// Storage index of metadata word w (K values [32w, 32w + 32)) of row r, for a
// weight of n rows with `words` = k / 32 words per row.  The words of a row
// are cut into blocks of 4 (128 values of K); block b holds every row's words
// of that block, row after row, and a last, narrower block does the same.  A
// K step of a row range is then one contiguous piece of the metadata, so the
// GEMM kernels load it in whole cache lines.
__host__ __device__ inline int64_t meta_index(int64_t r, int64_t w, int64_t n, int64_t words) {
  const int64_t b = w >> 2;
  const int64_t width = words - 4 * b < 4 ? words - 4 * b : 4;
  return 4 * n * b + r * width + (w & 3);
}

// sp24_format.hip
hipError_t launch_prune_compress(const uint16_t* w, int64_t n, int64_t k, uint16_t* values,
                                 uint32_t* meta, hipStream_t s);
hipError_t launch_decompress(int dtype, const void* values, const uint32_t* meta, int64_t n,
                             int64_t k, void* out, hipStream_t s);
hipError_t launch_check_meta(const uint32_t* meta, int64_t n, int64_t k, uint32_t* bad,
                             hipStream_t s);

// sp24_quant.hip
size_t quant_workspace_bytes(int64_t count);
hipError_t launch_slide_prune_pack(const uint16_t* w, int64_t n, int64_t k, int np, uint16_t* out,
                                   hipStream_t s);
// dtype SP24_FP8_E4M3 or SP24_INT8
hipError_t launch_slide_quant_rows(int dtype, const uint16_t* x, int64_t m, int64_t k, int np, uint8_t* q,
                                   float* scales, hipStream_t s);
// dtype SP24_FP8_E4M3 or SP24_INT8
hipError_t launch_quant_rows(int dtype, const uint16_t* x, int64_t m, int64_t k, uint8_t* q, float* scales,
                             hipStream_t s);
hipError_t launch_quant(int dtype, const uint16_t* x, int64_t count, uint8_t* q, float* scale, int mode,
                        void* ws, hipStream_t s);
// E4M3 codes with one scale per group of `group` values of a row ([rows, cols], cols % group == 0)
hipError_t launch_quant_groups(const uint16_t* x, int64_t rows, int64_t cols, int64_t group, uint8_t* q,
                               float* scales, hipStream_t s);

// sp24_palette.hip: the encoded exponent-palette weight (device pointers)
struct PaletteArgs {
  const uint8_t* palette;   // 16 exponents
  int64_t n_pal;            // rows in palette form
  const uint8_t* sm;        // [n_pal, k] sign+mantissa bytes
  const uint32_t* ix;       // [n_pal, k/8] index words
  const int32_t* pal_rows;  // [n_pal] row numbers
  int64_t n_verb;           // rows stored verbatim
  const uint16_t* verb;     // [n_verb, k] bf16
  const int32_t* verb_rows; // [n_verb] row numbers
};
constexpr int kPaletteWaves = 4;   // waves per workgroup of the small-m palette GEMM
constexpr int kPaletteRb1MaxM = 4; // up to this m one 16-row block per workgroup ...
constexpr int kPaletteRbWide = 2;  // ... above it this many blocks share a wave's X
constexpr int kPaletteXlMaxM = 1;        // X in LDS for m up to this ...
constexpr int kPaletteXLdsBytes = 61440;  // ... and X rows up to this size (with the
                                          // 4 KB reduction buffer, within 64 KB per workgroup)
constexpr int kPaletteMaxM = 16;   // largest m of the kernel that rebuilds BF16 in registers
size_t palette_analyze_ws_bytes(int64_t n);
hipError_t launch_palette_analyze(const uint16_t* w, int64_t n, int64_t k, uint8_t* palette, int32_t* slot,
                                  int32_t* counts, void* ws, hipStream_t s);
hipError_t launch_palette_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* palette, const int32_t* slot,
                               int64_t n_pal, int64_t n_verb, uint8_t* sm, uint32_t* ix, int32_t* pal_rows,
                               uint16_t* verb, int32_t* verb_rows, hipStream_t s);
hipError_t launch_palette_decode(const PaletteArgs& p, int64_t n, int64_t k, uint16_t* w, hipStream_t s);
hipError_t launch_palette_gemm_small(const uint16_t* x, const PaletteArgs& p, uint16_t* y, int m, int n, int k,
                                     hipStream_t s);

// sp24_gemm_skinny.hip / sp24_gemm_stream.hip / sp24_gemm_tiled.hip / sp24_reduce.hip
struct GemmArgs {
  int dtype;
  bool sparse;
  int m, n, k;
  const void* x;
  const float* x_scale;
  const void* w;        // compressed values (sparse) or dense W
  const uint32_t* meta; // sparse only
  const float* w_scale;
  uint16_t* y;
  float* partial;       // split-K partial sums [split_k][m][n], or nullptr
  // X quantised inside the GEMM (sparse FP8 stream kernel only): x_bf16 is X,
  // and the kernel writes the per-tensor scale to x_scale_out, which x_scale
  // then points to for the split-K reduction
  const uint16_t* x_bf16 = nullptr;
  float* x_scale_out = nullptr;
  // FP8: the scale of X row m is x_scale[m * x_scale_step] (0: one per tensor, 1: one per row)
  int x_scale_step = 0;
  // FP8: the scale of W row n is w_scale[n * w_scale_step] (0: one per tensor, 1: one per row)
  int w_scale_step = 0;
  // FP8 with scales per group of group_units units of 128 K (stream kernel only): X row m
  // and W row n carry n_groups scales each, x_gscale[m * n_groups + g] and
  // w_gscale[n * n_groups + g]; the kernel applies them to each unit's partial sums, so
  // the epilogue and the split-K reduction apply none (x_scale and w_scale unused)
  const float* x_gscale = nullptr;
  const float* w_gscale = nullptr;
  int group_units = 0;
  int n_groups = 0;
  // with x_bf16: one scale per token (written to x_scale_out[m]) instead of one per
  // tensor, and X rows lifted to the SlideSparse windows of N = x_lift (0: none)
  bool x_rows = false;
  int x_lift = 0;
};
// Small-m kernel configurations: X(id, row blocks of 16, token blocks of 16,
// waves per workgroup, chunks of loads issued per batch).
#define SP24_SKINNY_CONFIGS(X) \
  X(0, 1, 1, 8, 1)             \
  X(1, 1, 1, 4, 2)             \
  X(2, 1, 1, 2, 4)             \
  X(3, 2, 1, 4, 2)             \
  X(4, 2, 1, 8, 1)             \
  X(5, 4, 1, 4, 2)             \
  X(6, 2, 2, 8, 1)             \
  X(7, 2, 4, 4, 1)             \
  X(8, 4, 4, 4, 1)             \
  X(9, 4, 2, 4, 1)             \
  X(10, 1, 1, 4, 1)            \
  X(11, 2, 2, 4, 2)            \
  X(12, 1, 4, 4, 1)            \
  X(13, 2, 1, 2, 4)            \
  X(14, 1, 1, 8, 2)            \
  X(15, 4, 1, 8, 1)            \
  X(16, 1, 2, 8, 1)            \
  X(17, 2, 4, 8, 1)
constexpr int kSkinnyConfigs = 18;
constexpr int kTiledConfig = 99;     // config id of the LDS-tiled large-m kernel (256 x 256 tiles)
constexpr int kTiled128Config = 98;  // the same kernel with 128 W rows x 256 tokens (one-byte codes)

// Small-m LDS-ring kernel configurations (config id = kStreamBase + id):
// X(id, waves along n, row blocks of 16 per wave, waves along m, waves along
//   K, token blocks of 16 per wave, 128-K units per wave per step, LDS
//   buffers at most).  An entry runs an operand type only where two LDS
// buffers fit (stream_fits); the planner never picks it otherwise.
#define SP24_STREAM_CONFIGS(X)       \
  X(0, 4, 1, 1, 1, 1, 2, 6)          \
  X(1, 4, 1, 1, 2, 1, 1, 6)          \
  X(2, 4, 1, 1, 1, 4, 2, 4)          \
  X(3, 4, 1, 1, 2, 4, 1, 4)          \
  X(4, 1, 1, 1, 4, 1, 1, 6)          \
  X(5, 1, 1, 1, 8, 1, 1, 4)          \
  X(6, 1, 1, 1, 4, 4, 1, 3)          \
  X(7, 2, 1, 1, 2, 1, 1, 6)          \
  X(8, 2, 1, 1, 4, 2, 1, 3)          \
  X(9, 8, 1, 1, 1, 1, 2, 4)          \
  X(10, 4, 1, 1, 1, 2, 2, 4)         \
  X(11, 2, 1, 1, 2, 4, 1, 4)         \
  X(12, 8, 1, 1, 1, 4, 1, 3)         \
  X(13, 4, 1, 1, 2, 2, 1, 4)         \
  X(14, 1, 1, 1, 4, 2, 1, 4)         \
  X(15, 2, 1, 1, 4, 1, 1, 4)         \
  X(16, 4, 1, 1, 2, 1, 1, 10)        \
  X(17, 2, 1, 1, 4, 1, 1, 8)         \
  X(18, 4, 1, 1, 4, 1, 1, 6)         \
  X(19, 1, 1, 1, 8, 1, 1, 8)         \
  X(20, 2, 2, 1, 4, 4, 1, 3)         \
  X(21, 1, 8, 4, 1, 4, 1, 3)         \
  X(22, 1, 8, 8, 1, 2, 1, 3)         \
  X(23, 1, 4, 4, 1, 4, 1, 3)         \
  X(24, 1, 4, 8, 1, 2, 1, 3)         \
  X(25, 2, 4, 4, 1, 2, 1, 3)         \
  X(26, 1, 2, 8, 1, 2, 1, 4)         \
  X(27, 1, 4, 4, 2, 4, 1, 2)         \
  X(28, 8, 1, 1, 1, 4, 1, 8)         \
  X(29, 8, 1, 1, 1, 4, 2, 3)         \
  X(30, 2, 4, 4, 1, 2, 2, 3)
constexpr int kStreamConfigs = 31;
constexpr int kStreamBase = 100;
constexpr int kStreamLdsBytes = 160 * 1024;
// A stream kernel that quantises X itself holds its tokens' X codes for its K
// slice in dynamic LDS after its ring, sized per launch (rows * row bytes), so
// that a small region (M = 1) keeps the configuration's occupancy and a large
// one (M = 16 over K = 4096: 66 KB) takes what the ring leaves.  A
// configuration is a quantising one when at least kStreamQxMinBytes are left.
constexpr int kStreamQxMinBytes = 16384;

// Bytes of one LDS buffer of a stream configuration: W values and metadata of
// 16 * rbw * rb rows plus 16 * mw * mb X rows, for u * kw units of 128 K.
constexpr int stream_stage_bytes(int dtype, bool sparse, int rbw, int rb, int mw, int kw, int mb, int u) {
  const int esz = dtype == SP24_BF16 ? 2 : 1;
  const int ups = u * kw;
  const int wb = ups * (sparse ? 64 : 128) * esz, mwords = sparse ? ups * 4 : 0, xb = ups * 128 * esz;
  return 16 * rbw * rb * (wb + 4 * mwords) + 16 * mw * mb * xb;
}
// budget: LDS bytes the ring may take (less than the whole LDS when the kernel
// keeps a table of group scales beside it).
constexpr int stream_stages(int dtype, bool sparse, int rbw, int rb, int mw, int kw, int mb, int u,
                            int smax, int budget = kStreamLdsBytes) {
  const int fit = budget / stream_stage_bytes(dtype, sparse, rbw, rb, mw, kw, mb, u);
  return smax < fit ? smax : fit;
}
constexpr bool stream_fits(int dtype, bool sparse, int rbw, int rb, int mw, int kw, int mb, int u,
                           int smax, int budget = kStreamLdsBytes) {
  return stream_stages(dtype, sparse, rbw, rb, mw, kw, mb, u, smax, budget) >= 2;
}
// LDS bytes of a stream configuration below anything else: its ring or the
// reduction of the KW partial tiles, whichever is larger.  With qx (X
// quantised by the kernel itself and held in LDS) the ring buffers hold W and
// metadata only; the X rows live after these bytes.
constexpr int stream_ring_bytes(int dtype, bool sparse, int rbw, int rb, int mw, int kw, int mb, int u,
                                int smax, bool qx, int budget = kStreamLdsBytes) {
  const int esz = dtype == SP24_BF16 ? 2 : 1;
  const int stage = stream_stage_bytes(dtype, sparse, rbw, rb, mw, kw, mb, u) -
                    (qx ? 16 * mw * mb * u * kw * 128 * esz : 0);
  const int ring = stream_stages(dtype, sparse, rbw, rb, mw, kw, mb, u, smax, budget) * stage;
  const int red = kw > 1 ? kw * rbw * mw * rb * mb * 1024 : 0;
  return ring > red ? ring : red;
}
// Group scales (sp24_gemm_groups): the sparse FP8 stream kernel keeps the scales
// of its rows and tokens for its whole K slice in an LDS table of kStreamGsBytes
// beside its ring, as [group][row] and [group][token] fp32 arrays: (rows of the
// configuration + tokens of the configuration) * groups of the slice * 4 bytes
// must fit.  The ring then gets the rest of the LDS.
constexpr int kStreamGsBytes = 32768;
constexpr int kStreamGsBudget = kStreamLdsBytes - kStreamGsBytes;
constexpr bool stream_gs_fits(int rbw, int rb, int mw, int kw, int mb, int u, int smax) {
  return stream_fits(SP24_FP8_E4M3, true, rbw, rb, mw, kw, mb, u, smax, kStreamGsBudget) &&
         stream_ring_bytes(SP24_FP8_E4M3, true, rbw, rb, mw, kw, mb, u, smax, false, kStreamGsBudget) <=
             kStreamGsBudget;
}
// LDS bytes a quantising stream configuration (sparse FP8) leaves for its X
// codes: the LDS less its ring without X rows, the per-wave (per tensor) or
// per-row (per token) maxima and 256 bytes for the alignment of the static
// arrays; a configuration can quantise X itself when that is at least
// kStreamQxMinBytes.
constexpr int stream_qx_room(int rbw, int rb, int mw, int kw, int mb, int u, int smax, bool rows) {
  return kStreamLdsBytes - stream_ring_bytes(SP24_FP8_E4M3, true, rbw, rb, mw, kw, mb, u, smax, true) - 64 -
         (rows ? 4 * 16 * mw * mb : 0) - 256;
}
constexpr bool stream_qx_fits(int rbw, int rb, int mw, int kw, int mb, int u, int smax, bool rows) {
  return stream_fits(SP24_FP8_E4M3, true, rbw, rb, mw, kw, mb, u, smax) &&
         stream_qx_room(rbw, rb, mw, kw, mb, u, smax, rows) >= kStreamQxMinBytes;
}
// Row stride of the X rows a quantising stream kernel holds in LDS: its K
// slice, plus 128 bytes when that keeps 128-byte steps (one unit per step) on
// alternating bank halves as in a ring buffer.
constexpr int64_t stream_qx_row_bytes(int64_t k_slice, int step_bytes) {
  return k_slice + ((step_bytes == 128 && (k_slice / 128) % 2 == 0) ? 128 : 0);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, const sp24_plan& p, hipStream_t s);
hipError_t launch_gemm_stream(const GemmArgs& a, const sp24_plan& p, hipStream_t s);
hipError_t launch_gemm_tiled(const GemmArgs& a, const sp24_plan& p, hipStream_t s);
hipError_t launch_gemm_tiled128(const GemmArgs& a, const sp24_plan& p, hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs& a, int split_k, hipStream_t s);

// host plan (sp24_plan.cpp logic lives in sp24_api.hip)
int plan_gemm(int op, int dtype, int64_t m, int64_t n, int64_t k, sp24_plan* out);

}  // namespace sp24
