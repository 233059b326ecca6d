// C ABI of libsp24: argument validation, launch planning and dispatch.
//
// Every argument is checked before the first HIP call, so each error path can
// be exercised on a host without a GPU.  Launch planning (the choice of kernel,
// tile and K split from the sizes) is pure host logic and exported through
// sp24_plan_gemm.  The role it plays is that of the static shape profiles the
// cookbook page ("Deploying 2:4 Sparsity with FP8 on Hopper", "Engine
// integration and shape discipline") builds engines with, except that a shape
// outside the table is never silently sent to a dense kernel: every accepted
// shape runs the sparse kernels and every rejected one returns an error.
#include <limits.h>

#include <atomic>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// INT8 sums stay exact in int32: at most k products of magnitude <= 127 * 127
// per output (k/2 kept pairs for the sparse kernels), 16129 * 131072 < 2^31.
constexpr int64_t kMaxKInt8 = 131072;

bool known_dtype(int dtype) { return dtype == SP24_BF16 || dtype == SP24_FP8_E4M3 || dtype == SP24_INT8; }
bool scaled_dtype(int dtype) { return dtype == SP24_FP8_E4M3 || dtype == SP24_INT8; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool sync_check_enabled() {
  static const bool on = [] {
    const char* v = getenv("SP24_SYNC_CHECK");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

int finish(hipError_t launch, hipStream_t s) {
  if (launch != hipSuccess) return SP24_ERR_HIP;
  if (sync_check_enabled()) {
    if (hipStreamSynchronize(s) != hipSuccess) return SP24_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return SP24_ERR_HIP;
  }
  return SP24_OK;
}

int esize(int dtype) { return dtype == SP24_BF16 ? 2 : 1; }

// SP24_TILE="config,split_k[,rows]" overrides the small-m plan (tuning and
// tests only): split_k 0 keeps the automatic choice; rows (stream kernel
// only) sets the rows per workgroup.
bool tile_override(int* cfg, int* sk, int* rows) {
  const char* v = getenv("SP24_TILE");
  if (v == nullptr || v[0] == '\0') return false;
  int a, b, r = 0;
  const int got = sscanf(v, "%d,%d,%d", &a, &b, &r);
  if (got < 2) return false;
  const bool known = (a >= 0 && a < kSkinnyConfigs) || a == kTiledConfig || a == kTiled128Config ||
                     (a >= kStreamBase && a < kStreamBase + kStreamConfigs);
  if (!known || b < 0 || b > 64 || r < 0) return false;
  *cfg = a;
  *sk = b;
  *rows = got == 3 ? r : 0;
  return true;
}

struct Cfg {
  int rb, mb, nw, batch;
};

struct StreamShape {
  int rbw, rb, mw, kw, mb, u, smax;
};

struct StreamChoice {
  int id;
  int64_t rows;
  int split_k = 0;  // 0: automatic
};

StreamShape stream_shape(int id) {
  switch (id) {
#define SP24_STREAM_SHAPE(ID, RBW, RB, MW, KW, MB, U, SMAX) \
  case ID: return StreamShape{RBW, RB, MW, KW, MB, U, SMAX};
    SP24_STREAM_CONFIGS(SP24_STREAM_SHAPE)
#undef SP24_STREAM_SHAPE
  }
  return StreamShape{1, 1, 1, 1, 1, 1, 2};
}

// Plan of stream configuration `id` (0-based) for a shape, or false if the
// configuration cannot run it (K must split into whole steps, and two LDS
// buffers of the operand type must fit).  Each
// workgroup takes one range of rows: the rows are shared equally over about
// 256 workgroups per token block (a multiple of 4 rows, at least 16, at most
// the configuration's row blocks), so every CU streams the same amount of W.
// split_k 0 picks the split automatically: K is split over the grid only when
// the row ranges alone leave more than half of the CUs idle.
bool plan_stream(int id, int dtype, bool sparse, int sk_req, int rows_req, int64_t m, int64_t n,
                 int64_t k, sp24_plan* out) {
  const StreamShape c = stream_shape(id);
  if (!stream_fits(dtype, sparse, c.rbw, c.rb, c.mw, c.kw, c.mb, c.u, c.smax)) return false;
  const int64_t bn = 16 * c.rbw * c.rb, bm = 16 * c.mw * c.mb, ups = (int64_t)c.u * c.kw;
  const int64_t units = k / 128;
  if (units % ups != 0) return false;
  const int64_t gy = (m + bm - 1) / bm;
  if (gy > 65535) return false;
  const int64_t shares = gy >= 256 ? 1 : 256 / gy;
  int64_t rows = ((n + shares - 1) / shares + 3) / 4 * 4;
  rows = rows < 16 ? 16 : rows;  // below one row block, split K instead: X is re-read per range
  rows = rows < bn ? rows : bn;
  if (rows_req > 0) {
    if (rows_req % 4 != 0 || rows_req > bn) return false;
    rows = rows_req;
  }
  const int64_t gx = (n + rows - 1) / rows;
  if (gx > INT_MAX) return false;
  int64_t sk = sk_req > 0 ? sk_req : 1;
  if (sk_req == 0)
    while (sk < 16 && gx * gy * sk * 2 <= 256 && units % (2 * sk * ups) == 0) sk *= 2;
  if (units % (sk * ups) != 0 || sk > 65535) return false;
  out->kernel = SP24_KERNEL_STREAM;
  out->tile_n = (int)rows;
  out->tile_m = (int)bm;
  out->waves = c.rbw * c.mw * c.kw;
  out->split_k = (int)sk;
  out->grid_x = (int)gx;
  out->grid_y = (int)gy;
  out->grid_z = (int)sk;
  out->config = kStreamBase + id;
  out->batch = c.u;
  out->workspace_bytes = sk > 1 ? (size_t)sk * (size_t)m * (size_t)n * sizeof(float) : 0;
  return true;
}

// Default stream configuration and rows per workgroup for a shape (rows 0:
// equal shares over ~256 workgroups per token block).  Chosen from sweeps of
// every configuration on the decode shapes of a Llama-3-8B-sized layer on
// MI355X:
//  * m <= 16: X is negligible and W streams at the HBM rate; short row ranges
//    want many waves along K (4 waves over 16 rows: down-projection 4096 x 14336
//    at m = 1 / 16 8.3 / 10.2 against 8.6 / 10.8 us with 8; the calls that
//    quantise X inside the kernel take 8, plan_qx below), ~30-64 rows per CU do
//    best as two 8-wave workgroups per CU at m <= 8 and as one workgroup of 4
//    row blocks x 32 tokens at 8 < m <= 16 (up-projection at m = 16: 8.65
//    against 9.2 us), longer ranges as 8 row blocks.
//    BF16 (twice the bytes per step, so the two-workgroup ring no longer fits
//    twice in a CU's LDS) does best there with one workgroup of 4 x 16 rows
//    per CU (up-projection, 14336 x 4096: 15.7 against 16.3 us at m = 1, 15.8
//    against 17.4 us at m = 16).
//  * m <= 64: X (m*k bytes per workgroup, from L2 into LDS) costs as much as
//    W's share when a CU has few rows, so few-row shapes take 32 tokens per
//    workgroup (W read twice, the second time from cache), or, for long K, 64
//    rows per workgroup with K split over 4 workgroups.
//  * m <= 256: wide shapes (more than 64 rows per CU) keep all 256 tokens in
//    one workgroup with 8 waves along m, so that W streams once (gate+up,
//    28672 x 4096 at m = 256, FP8: 38.5 us against 40.6 us for the tiled
//    kernel); long-K few-row shapes take 128 rows x 128 tokens per workgroup
//    with K split in 4 (down-projection 4096 x 14336: 27.0 against 29.5 us
//    for 64 rows x 256 tokens); the rest take 64-token blocks.
//  * Sparse one-byte codes at m <= 256 with 128-row workgroups step two units
//    of K at a time (W in 128-byte row pieces; one unit moves 64-byte halves of
//    a line, which the load path takes at half the rate): QKV 6144 x 4096 at
//    m = 256 15.0 against 16.3 us, down 4096 x 14336 26.4 against 27.4 us.
StreamChoice stream_default(int dtype, bool sparse, int64_t m, int64_t n, int64_t k) {
  const bool two_units = sparse && dtype != SP24_BF16;
  const int64_t rows_cu = (n + 255) / 256;
  auto rows_for = [&](int64_t shares, int64_t lo, int64_t hi) {
    int64_t r = ((n + shares - 1) / shares + 3) / 4 * 4;
    return r < lo ? lo : (r > hi ? hi : r);
  };
  if (m <= 16) {
    if (rows_cu <= 16) return StreamChoice{4, 0};
    if (rows_cu <= 64) {
      if (dtype == SP24_BF16) return rows_cu > 32 ? StreamChoice{13, 0} : StreamChoice{15, rows_for(256, 16, 32)};
      if (m > 8 && rows_cu > 32) return StreamChoice{10, rows_for(256, 16, 64)};
      return StreamChoice{15, rows_for(rows_cu <= 32 ? 256 : 512, 16, 32)};
    }
    return StreamChoice{9, 0};
  }
  if (m <= 32) {
    if (rows_cu <= 16) return StreamChoice{14, 0};
    if (rows_cu <= 64) return StreamChoice{8, rows_for(rows_cu <= 32 ? 256 : 512, 16, 32)};
    return StreamChoice{13, 0};
  }
  if (m <= 64) {
    if (rows_cu <= 16) return k >= 8192 ? StreamChoice{3, 64} : StreamChoice{8, 0};
    if (rows_cu <= 32) return StreamChoice{13, 0};
    if (rows_cu <= 64) return StreamChoice{3, 0};
    return StreamChoice{12, 0};
  }
  if (m <= 256) {
    // 256 tokens per workgroup (8 waves along m): W is streamed once
    if (rows_cu > 64) return StreamChoice{22, 0};
    if (rows_cu <= 16 && k >= 8192) return StreamChoice{two_units ? 30 : 25, 128, 4};
  }
  // 64-token blocks: more than 64 rows per share take 128-row workgroups, with an
  // 8-buffer ring for one unit per step (QKV 6144 x 4096 at m = 256: 15.5 against
  // 16.5 us with 3 buffers)
  const int64_t gy = (m + 63) / 64;
  const int64_t shares = gy >= 256 ? 1 : 256 / gy;
  if ((n + shares - 1) / shares > 64) return StreamChoice{two_units ? 29 : 28, 0};
  return StreamChoice{3, 0};
}

Cfg skinny_cfg(int id) {
  switch (id) {
#define SP24_CFG_CASE(ID, RB, MB, NW, BATCH) \
  case ID: return Cfg{RB, MB, NW, BATCH};
    SP24_SKINNY_CONFIGS(SP24_CFG_CASE)
#undef SP24_CFG_CASE
  }
  return Cfg{1, 1, 8, 1};
}

// K split of the LDS-tiled kernel (256 x 256 tiles): 1 without a split, 0 when the
// tiled kernel is not the plan, negative when a requested split is invalid.
// K slices are whole steps (128 values for one-byte codes, 64 for bf16), an even
// number of them (bf16 metadata steps come in pairs of words), at most 64 slices.
// req >= 0: the split asked for through SP24_TILE (0: automatic); req < 0: the
// automatic choice.  It takes the tiled kernel for m > 256 with at least 128 tiles,
// and for BF16 at 128 < m <= 256 (one tile of tokens) with at least 96 tiles, where
// the 256-token stream configurations do not fit the LDS with two-byte operands
// (gate+up 28672 x 4096 at m = 256: 65 us with K split in two against 104 us for
// 64-token blocks).  One-byte codes keep the stream kernel there (FP8 gate+up: 38.5
// us against 40.6 us for the tiled kernel).  Fewer tiles leave CUs idle and the
// small-m kernels win (QKV, O, down of the same layer: 1.5-3x).
constexpr int64_t kTiled128MinTiles = 192;

int tiled_split(int dtype, bool sparse, int64_t m, int64_t n, int64_t k, int64_t tiles, int req) {
  (void)n;
  (void)sparse;
  const int64_t steps = k / (dtype == SP24_BF16 ? 64 : 128);
  auto valid = [&](int64_t s) { return s >= 1 && s <= 64 && steps % s == 0 && (s == 1 || (steps / s) % 2 == 0); };
  if (req > 0) return valid(req) ? (int)req : -1;
  if (req == 0) return 1;
  if (m > 256 && tiles >= 128) return 1;
  if (m > 128 && m <= 256 && tiles >= 96 && dtype == SP24_BF16) return valid(2) ? 2 : 1;
  return 0;
}

}  // namespace

int plan_gemm(int op, int dtype, int64_t m, int64_t n, int64_t k, sp24_plan* out) {
  if (out == nullptr) return SP24_ERR_NULL;
  memset(out, 0, sizeof(*out));
  if (op != SP24_OP_GEMM && op != SP24_OP_DENSE_GEMM) return SP24_ERR_MODE;
  if (!known_dtype(dtype)) return SP24_ERR_DTYPE;
  if (m < 1 || n < 1 || k < 128 || k % 128 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim)
    return SP24_ERR_SHAPE;
  if (dtype == SP24_INT8 && k > kMaxKInt8) return SP24_ERR_SHAPE;

  // Large m with enough 256 x 256 tiles to fill the chip: LDS-tiled kernel.  One
  // tile of tokens (128 < m <= 256) over a wide layer with one-byte codes: the same
  // kernel with 128-row tiles when those number at least kTiled128MinTiles (gate+up
  // 28672 x 4096 at m = 256, FP8: 34.4 us for 224 tiles of 128 rows against 43.8 us
  // for the stream kernel with all 256 tokens per workgroup and 40.6 us for 112
  // tiles of 256 rows); narrower layers keep the stream kernel (QKV, O and down of
  // the same layer: 22-33 us with 128-row tiles against 11.6-28 us).
  const int64_t tiles = ((n + 255) / 256) * ((m + 255) / 256);
  const int64_t tiles128 = ((n + 127) / 128) * ((m + 255) / 256);
  int id, sk = 0;
  if (m <= 16) {
    id = n >= 8192 ? 5 : 1;
  } else if (m <= 32) {
    id = 11;
  } else if (m <= 64) {
    id = n >= 8192 ? 8 : 11;
  } else {
    id = 8;
  }
  int oid, osk, orows = 0;
  const bool forced = tile_override(&oid, &osk, &orows);
  if (forced) {
    id = oid;
    sk = osk;
  }
  const bool one_byte = dtype != SP24_BF16;
  const bool auto128 = !forced && one_byte && m > 128 && m <= 256 && tiles128 >= kTiled128MinTiles;
  const bool use128 = auto128 || (forced && id == kTiled128Config);
  if (use128 && !one_byte) return SP24_ERR_SHAPE;
  const bool tiled_req = forced && (id == kTiledConfig || id == kTiled128Config);
  const int tsk = auto128 ? 1
                          : tiled_split(dtype, op == SP24_OP_GEMM, m, n, k, use128 ? tiles128 : tiles,
                                        tiled_req ? sk : -1);
  if ((!forced && tsk > 0) || tiled_req) {
    const int64_t t = use128 ? tiles128 : tiles;
    if (t > INT_MAX || tsk < 1) return SP24_ERR_SHAPE;
    out->kernel = SP24_KERNEL_TILED;
    out->tile_n = use128 ? 128 : 256;
    out->tile_m = 256;
    out->waves = 8;
    out->split_k = tsk;
    out->grid_x = (int)t;
    out->grid_y = tsk;
    out->grid_z = 1;
    out->config = use128 ? kTiled128Config : kTiledConfig;
    out->batch = 1;
    out->workspace_bytes = tsk > 1 ? (size_t)tsk * (size_t)m * (size_t)n * sizeof(float) : 0;
    return SP24_OK;
  }
  if (forced && id >= kStreamBase) {
    if (!plan_stream(id - kStreamBase, dtype, op == SP24_OP_GEMM, sk, orows, m, n, k, out))
      return SP24_ERR_SHAPE;
    return SP24_OK;
  }
  if (!forced) {
    // the choice for this shape, else (it does not fit this operand type, or K
    // does not split into its steps) the 64-token-block configurations
    const StreamChoice d = stream_default(dtype, op == SP24_OP_GEMM, m, n, k);
    if (plan_stream(d.id, dtype, op == SP24_OP_GEMM, d.split_k, (int)d.rows, m, n, k, out)) return SP24_OK;
    const int64_t gy = (m + 63) / 64, shares = gy >= 256 ? 1 : 256 / gy;
    const int g = (n + shares - 1) / shares > 64 ? 12 : 3;
    if (m > 64 && plan_stream(g, dtype, op == SP24_OP_GEMM, 0, 0, m, n, k, out)) return SP24_OK;
  }
  const Cfg c = skinny_cfg(id);
  const int tn = 16 * c.rb, tm = 16 * c.mb, nw = c.nw;
  const int64_t gx = (n + tn - 1) / tn, gy = (m + tm - 1) / tm;
  const int64_t chunks = (k / 128 + 3) / 4;
  if (sk == 0) {
    // Split K over the grid only when the tiles alone leave CUs idle and each
    // wave keeps at least two chunks of K.
    sk = 1;
    while (sk < 8 && gx * gy * sk < 256 && chunks >= (int64_t)nw * sk * 2 * 2) sk *= 2;
  }
  if (gx > INT_MAX || gy > 65535) return SP24_ERR_SHAPE;
  out->kernel = SP24_KERNEL_SKINNY;
  out->tile_n = tn;
  out->tile_m = tm;
  out->waves = nw;
  out->split_k = sk;
  out->grid_x = (int)gx;
  out->grid_y = (int)gy;
  out->grid_z = sk;
  out->config = id;
  out->batch = c.batch;
  out->workspace_bytes = sk > 1 ? (size_t)sk * (size_t)m * (size_t)n * sizeof(float) : 0;
  return SP24_OK;
}

namespace {

// Plan of sp24_gemm_groups with group scales finer than one per row (group < k):
// the sparse FP8 stream kernel with its table of group scales (stream_gs_fits),
// sized for 128-K groups, so that one plan (and one workspace size) serves every
// group: the default stream configuration of the shape when it is a stream plan
// that fits and holds at most 8 tiles per wave (two sets of unscaled tiles are
// kept besides the accumulators), else the 64-token, 128-row configuration of one
// unit per step (config 12, which takes any k % 128 == 0); K is split further
// while the scales of a slice, (rows + tokens) * units * 4 bytes, exceed the
// table.
int plan_groups(int64_t m, int64_t n, int64_t k, sp24_plan* out) {
  sp24_plan p;
  int st = plan_gemm(SP24_OP_GEMM, SP24_FP8_E4M3, m, n, k, &p);
  if (st != SP24_OK) return st;
  const int64_t units = k / 128;
  auto fits = [&](int id) {
    const StreamShape c = stream_shape(id);
    return stream_gs_fits(c.rbw, c.rb, c.mw, c.kw, c.mb, c.u, c.smax) && c.u * c.rb * c.mb <= 8;
  };
  const int ids[2] = {p.kernel == SP24_KERNEL_STREAM ? p.config - kStreamBase : -1, 12};
  for (int id : ids) {
    if (id < 0 || !fits(id)) continue;
    const StreamShape c = stream_shape(id);
    const int64_t ups = (int64_t)c.u * c.kw, table = 16 * (c.rbw * c.rb + c.mw * c.mb) * 4;
    const int rows = id == ids[0] ? p.tile_n : 0;
    int sk = id == ids[0] ? p.split_k : 1;
    while (table * (units / sk) > kStreamGsBytes && units % (2 * sk * ups) == 0 && sk < 64) sk *= 2;
    if (table * (units / sk) > kStreamGsBytes) continue;
    if (plan_stream(id, SP24_FP8_E4M3, true, sk, rows, m, n, k, out)) return SP24_OK;
  }
  return SP24_ERR_SHAPE;
}

// X quantised inside the GEMM (sp24_gemm_qx, sp24_gemm_rows_qx,
// sp24_slide_gemm_qx): the sparse FP8 stream kernel holds the codes of a
// workgroup's tokens over its K slice in dynamic LDS after its ring, as much as
// the ring leaves (stream_qx_room).  With one scale per tensor every workgroup
// also reads all of X for it, so X must be small (M * K <= kQxMaxValues, 128 KB
// of bf16); with one scale per token a workgroup reads only its own tokens.
// Every workgroup reads and casts all of its tokens' K slice, repeated by every
// workgroup along n: it is fused only while that is at most kQxMaxWgValues
// values per workgroup (one token over K = 14336, four over K = 4096).
// Measured on MI355X, the up-projection 14336 x 4096 at m = 16 (65536 values
// per workgroup): 21.0 us fused against 12.9 us for the one-launch quantiser
// followed by the GEMM (the reading of X twice per workgroup, not the cast,
// sets the fused time).
constexpr int64_t kQxMaxValues = 65536;
constexpr int64_t kQxMaxWgValues = 16384;

// SP24_QX_FUSE=<values> replaces kQxMaxWgValues (tuning and tests only).
int64_t qx_max_wg_values() {
  const char* v = getenv("SP24_QX_FUSE");
  long long x = 0;
  if (v != nullptr && sscanf(v, "%lld", &x) == 1 && x >= 0 && x <= kQxMaxValues * 4) return x;
  return kQxMaxWgValues;
}

bool qx_fused(const sp24_plan& p, int64_t m, int64_t k, bool rows) {
  if (p.kernel != SP24_KERNEL_STREAM || (!rows && m * k > kQxMaxValues)) return false;
  int64_t room = -1;
  int ups = 0, bm = 0;
  switch (p.config - kStreamBase) {
#define SP24_QX_ROOM(ID, RBW, RB, MW, KW, MB, U, SMAX)                               \
  case ID:                                                                     \
    ups = (U) * (KW);                                                          \
    bm = 16 * (MW) * (MB);                                                     \
    if (stream_qx_fits(RBW, RB, MW, KW, MB, U, SMAX, rows)) room = stream_qx_room(RBW, RB, MW, KW, MB, U, SMAX, rows); \
    break;
    SP24_STREAM_CONFIGS(SP24_QX_ROOM)
#undef SP24_QX_ROOM
    default: return false;
  }
  const int64_t rows_wg = m < bm ? m : bm;
  return room >= 0 && rows_wg * (k / p.split_k) <= qx_max_wg_values() &&
         rows_wg * stream_qx_row_bytes(k / p.split_k, ups * 128) <= room;
}

// The plan of the calls that quantise X (sp24_gemm_qx, sp24_gemm_rows_qx,
// sp24_slide_gemm_qx): plan_gemm's, except that the 16-row, 4-K-wave plan of few
// rows per CU (config 104) becomes its 8-K-wave form (config 105) when X is then
// quantised inside the kernel: the prologue's cast runs on twice the waves
// (down-projection 4096 x 14336 at m = 1: 10.2 against 10.6 us per tensor),
// while the GEMM on codes is faster with 4.  A plan forced through SP24_TILE is
// kept as it is.
int plan_qx(int64_t m, int64_t n, int64_t k, bool rows, sp24_plan* out) {
  const int st = plan_gemm(SP24_OP_GEMM, SP24_FP8_E4M3, m, n, k, out);
  int cfg, sk, orows;
  if (st != SP24_OK || out->kernel != SP24_KERNEL_STREAM || out->config != kStreamBase + 4 ||
      tile_override(&cfg, &sk, &orows))
    return st;
  sp24_plan q;
  memset(&q, 0, sizeof(q));
  if (plan_stream(5, SP24_FP8_E4M3, true, out->split_k, 0, m, n, k, &q) && q.split_k == out->split_k &&
      q.workspace_bytes == out->workspace_bytes && qx_fused(q, m, k, rows))
    *out = q;
  return SP24_OK;
}

// Workspace of the quantising GEMMs: the GEMM's own, then (when X is not
// quantised inside the kernel) the E4M3 codes of X and, per tensor, the
// quantiser's workspace.  k is the GEMM's K (K' for SlideSparse).
struct QxWorkspace {
  size_t gemm, codes, quant, total;
  bool fused;
};

QxWorkspace qx_workspace(const sp24_plan& p, int64_t m, int64_t k, bool rows) {
  QxWorkspace w;
  w.gemm = (p.workspace_bytes + 15) / 16 * 16;
  w.fused = qx_fused(p, m, k, rows);
  w.codes = w.fused ? 0 : ((size_t)(m * k) + 15) / 16 * 16;
  w.quant = w.fused || rows ? 0 : quant_workspace_bytes(m * k);
  w.total = w.gemm + w.codes + w.quant;
  return w;
}

hipError_t launch_plan(const GemmArgs& a, const sp24_plan& p, hipStream_t s) {
  hipError_t e = p.kernel == SP24_KERNEL_TILED    ? (p.tile_n == 128 ? launch_gemm_tiled128(a, p, s)
                                                                     : launch_gemm_tiled(a, p, s))
                 : p.kernel == SP24_KERNEL_STREAM ? launch_gemm_stream(a, p, s)
                                                  : launch_gemm_skinny(a, p, s);
  if (e == hipSuccess && p.split_k > 1) e = launch_splitk_reduce(a, p.split_k, s);
  return e;
}

// Workspace of sp24_palette_gemm: none for m <= kPaletteMaxM; otherwise the
// rebuilt W (bf16) and the dense GEMM's own workspace after it.
struct PaletteWs {
  size_t weight, gemm, total;
  bool ok;
  sp24_plan plan;
};

PaletteWs palette_gemm_ws(int64_t m, int64_t n, int64_t k) {
  PaletteWs w{0, 0, 0, false, {}};
  if (m < 1 || n < 1 || k < 128 || k % 128 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim) return w;
  w.ok = true;
  if (m <= kPaletteMaxM) return w;
  if (plan_gemm(SP24_OP_DENSE_GEMM, SP24_BF16, m, n, k, &w.plan) != SP24_OK) {
    w.ok = false;
    return w;
  }
  w.weight = ((size_t)n * (size_t)k * 2 + 255) / 256 * 256;
  w.gemm = w.plan.workspace_bytes;
  w.total = w.weight + w.gemm;
  return w;
}

// Checks of an encoded palette weight of n rows: SP24_OK or the error.
int check_palette(const sp24_palette_weight* pw, int64_t n) {
  if (pw == nullptr || pw->palette == nullptr) return SP24_ERR_NULL;
  if (pw->n_pal < 0 || pw->n_verb < 0 || pw->n_pal + pw->n_verb != n) return SP24_ERR_SHAPE;
  if (pw->n_pal > 0 && (!pw->sm || !pw->ix || !pw->pal_rows)) return SP24_ERR_NULL;
  if (pw->n_verb > 0 && (!pw->verb || !pw->verb_rows)) return SP24_ERR_NULL;
  if (!aligned16(pw->palette)) return SP24_ERR_ALIGN;
  if (pw->n_pal > 0 && (!aligned16(pw->sm) || !aligned16(pw->ix) || ((uintptr_t)pw->pal_rows & 3u)))
    return SP24_ERR_ALIGN;
  if (pw->n_verb > 0 && (!aligned16(pw->verb) || ((uintptr_t)pw->verb_rows & 3u))) return SP24_ERR_ALIGN;
  return SP24_OK;
}

// Does an output of `bytes` at `out` overlap any array of the encoded weight?
// Rows of each kind are stored in blocks of 16 (the last one padded).
size_t pad16(int64_t rows) { return (size_t)((rows + 15) / 16 * 16); }

bool overlaps_palette(const void* out, size_t bytes, const sp24_palette_weight* pw, int64_t k) {
  if (overlaps(out, bytes, pw->palette, 16)) return true;
  if (pw->n_pal > 0 &&
      (overlaps(out, bytes, pw->sm, pad16(pw->n_pal) * k) || overlaps(out, bytes, pw->ix, pad16(pw->n_pal) * k / 2) ||
       overlaps(out, bytes, pw->pal_rows, (size_t)pw->n_pal * 4)))
    return true;
  if (pw->n_verb > 0 && (overlaps(out, bytes, pw->verb, pad16(pw->n_verb) * k * 2) ||
                         overlaps(out, bytes, pw->verb_rows, (size_t)pw->n_verb * 4)))
    return true;
  return false;
}

PaletteArgs palette_args(const sp24_palette_weight* pw) {
  PaletteArgs a;
  a.palette = pw->palette;
  a.n_pal = pw->n_pal;
  a.sm = pw->sm;
  a.ix = pw->ix;
  a.pal_rows = pw->pal_rows;
  a.n_verb = pw->n_verb;
  a.verb = static_cast<const uint16_t*>(pw->verb);
  a.verb_rows = pw->verb_rows;
  return a;
}

// Scratch memory of sp24_gemm_qx_noalloc, for callers that cannot allocate:
// one array per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is a stand-in, not a device
// address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kScratchBytes = SP24_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (the first call on a device looks it up).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return SP24_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SP24_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SP24_OK;
}

// sp24_gemm_qx (the caller's workspace) and sp24_gemm_qx_noalloc (use_scratch:
// this device's scratch array).  Every argument is checked before the first
// HIP call; with use_scratch the first HIP call is the scratch lookup.
int gemm_qx_common(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scale_dev,
                   const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                   void* ws, size_t ws_bytes, bool use_scratch, void* stream) {
  if (!x_bf16 || !x_scale_dev || !w_values || !w_meta || !w_scale_dev || !y_bf16) return SP24_ERR_NULL;
  sp24_plan p;
  int st = plan_qx(m, n, k, false, &p);
  if (st != SP24_OK) return st;
  if (!aligned16(x_bf16) || !aligned16(w_values) || !aligned16(w_meta) || !aligned16(y_bf16))
    return SP24_ERR_ALIGN;
  if (((uintptr_t)x_scale_dev & 3u) || ((uintptr_t)w_scale_dev & 3u)) return SP24_ERR_ALIGN;
  const QxWorkspace wsp = qx_workspace(p, m, k, false);
  if (use_scratch) {
    if (wsp.total > kScratchBytes) return SP24_ERR_WORKSPACE;
  } else if (wsp.total > 0) {
    if (ws == nullptr || ws_bytes < wsp.total) return SP24_ERR_WORKSPACE;
    if (!aligned16(ws)) return SP24_ERR_ALIGN;
  }
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 2, wb = (size_t)n * (k / 2);
  const size_t mb = (size_t)n * (k / 32) * 4;
  const void* in[4] = {x_bf16, w_values, w_meta, w_scale_dev};
  const size_t inb[4] = {xb, wb, mb, 4};
  for (int i = 0; i < 4; ++i)
    if (overlaps(y_bf16, yb, in[i], inb[i]) || overlaps(x_scale_dev, 4, in[i], inb[i]) ||
        (!use_scratch && wsp.total > 0 && overlaps(ws, wsp.total, in[i], inb[i])))
      return SP24_ERR_ALIAS;
  if (overlaps(y_bf16, yb, x_scale_dev, 4) ||
      (!use_scratch && wsp.total > 0 &&
       (overlaps(ws, wsp.total, y_bf16, yb) || overlaps(ws, wsp.total, x_scale_dev, 4))))
    return SP24_ERR_ALIAS;
  if (use_scratch && wsp.total > 0) {
    const int st2 = scratch_of_current_device(&ws);
    if (st2 != SP24_OK) return st2;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  GemmArgs a;
  a.dtype = SP24_FP8_E4M3;
  a.sparse = true;
  a.m = (int)m;
  a.n = (int)n;
  a.k = (int)k;
  a.x_scale = x_scale_dev;
  a.w = w_values;
  a.meta = w_meta;
  a.w_scale = w_scale_dev;
  a.y = static_cast<uint16_t*>(y_bf16);
  a.partial = p.split_k > 1 ? reinterpret_cast<float*>(wsb) : nullptr;
  if (wsp.fused) {
    a.x = nullptr;
    a.x_bf16 = static_cast<const uint16_t*>(x_bf16);
    a.x_scale_out = x_scale_dev;
    return finish(launch_plan(a, p, s), s);
  }
  uint8_t* codes = wsb + wsp.gemm;
  hipError_t e = launch_quant(SP24_FP8_E4M3, static_cast<const uint16_t*>(x_bf16), m * k, codes,
                              x_scale_dev, SP24_SCALE_DYNAMIC, wsp.quant > 0 ? codes + wsp.codes : nullptr, s);
  a.x = codes;
  if (e == hipSuccess) e = launch_plan(a, p, s);
  return finish(e, s);
}

}  // namespace

}  // namespace sp24

using namespace sp24;

extern "C" {

int sp24_version(void) { return SP24_VERSION; }

const char* sp24_status_string(int status) {
  switch (status) {
    case SP24_OK: return "ok";
    case SP24_ERR_NULL: return "a required pointer is NULL";
    case SP24_ERR_SHAPE: return "a size is out of range";
    case SP24_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case SP24_ERR_DTYPE: return "unknown dtype";
    case SP24_ERR_WORKSPACE: return "workspace missing or too small";
    case SP24_ERR_HIP: return "HIP launch or kernel failure";
    case SP24_ERR_MODE: return "unknown scale mode or op";
    case SP24_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
  }
}

int sp24_plan_gemm(int op, int dtype, int64_t m, int64_t n, int64_t k, sp24_plan* out) {
  return plan_gemm(op, dtype, m, n, k, out);
}

size_t sp24_workspace_size(int op, int dtype, int64_t m, int64_t n, int64_t k) {
  if (op == SP24_OP_QUANT) {
    // For the quantiser the element count is m * k (n is ignored); dtype must be BF16 input.
    (void)dtype;
    if (m < 1 || k < 1) return 0;
    return quant_workspace_bytes(m * k);
  }
  if (op == SP24_OP_PALETTE_ANALYZE) {
    if (n < 1 || k < 128 || k % 128 != 0 || n > kMaxDim || k > kMaxDim) return 0;
    return palette_analyze_ws_bytes(n);
  }
  if (op == SP24_OP_PALETTE_GEMM) return palette_gemm_ws(m, n, k).total;
  if (op == SP24_OP_GEMM_GROUPS) {
    // the larger of the two plans: one group per row (plan_gemm), finer groups (plan_groups)
    sp24_plan a, b;
    if (dtype != SP24_FP8_E4M3 || plan_gemm(SP24_OP_GEMM, dtype, m, n, k, &a) != SP24_OK ||
        plan_groups(m, n, k, &b) != SP24_OK)
      return 0;
    return a.workspace_bytes > b.workspace_bytes ? a.workspace_bytes : b.workspace_bytes;
  }
  sp24_plan p;
  if (op == SP24_OP_GEMM_QX || op == SP24_OP_GEMM_ROWS_QX) {
    if (dtype != SP24_FP8_E4M3 || plan_qx(m, n, k, op == SP24_OP_GEMM_ROWS_QX, &p) != SP24_OK) return 0;
    return qx_workspace(p, m, k, op == SP24_OP_GEMM_ROWS_QX).total;
  }
  if (plan_gemm(op, dtype, m, n, k, &p) != SP24_OK) return 0;
  return p.workspace_bytes;
}

int sp24_prune_compress(const void* w_bf16, int64_t n, int64_t k, void* values_bf16,
                        uint32_t* meta, void* stream) {
  if (!w_bf16 || !values_bf16 || !meta) return SP24_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0 || n > kMaxDim || k > kMaxDim) return SP24_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(values_bf16) || !aligned16(meta)) return SP24_ERR_ALIGN;
  const size_t wb = (size_t)n * k * 2, vb = wb / 2, mb = (size_t)n * (k / 32) * 4;
  if (overlaps(w_bf16, wb, values_bf16, vb) || overlaps(w_bf16, wb, meta, mb) ||
      overlaps(values_bf16, vb, meta, mb))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_prune_compress(static_cast<const uint16_t*>(w_bf16), n, k,
                                      static_cast<uint16_t*>(values_bf16), meta, s),
                s);
}

int sp24_decompress(int dtype, const void* values, const uint32_t* meta, int64_t n, int64_t k,
                    void* w_out, void* stream) {
  if (!known_dtype(dtype)) return SP24_ERR_DTYPE;
  if (!values || !meta || !w_out) return SP24_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0 || n > kMaxDim || k > kMaxDim) return SP24_ERR_SHAPE;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(w_out)) return SP24_ERR_ALIGN;
  const size_t ob = (size_t)n * k * esize(dtype), vb = ob / 2, mb = (size_t)n * (k / 32) * 4;
  if (overlaps(w_out, ob, values, vb) || overlaps(w_out, ob, meta, mb)) return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_decompress(dtype, values, meta, n, k, w_out, s), s);
}

int sp24_check_meta(const uint32_t* meta, int64_t n, int64_t k, uint32_t* bad_dev, void* stream) {
  if (!meta || !bad_dev) return SP24_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0 || n > kMaxDim || k > kMaxDim) return SP24_ERR_SHAPE;
  if (!aligned16(meta) || ((uintptr_t)bad_dev & 3u)) return SP24_ERR_ALIGN;
  if (overlaps(bad_dev, 4, meta, (size_t)n * (k / 32) * 4)) return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_check_meta(meta, n, k, bad_dev, s), s);
}

static int quant_common(int dtype, const void* x_bf16, int64_t count, uint8_t* q_out, float* scale_dev,
                        int mode, void* ws, size_t ws_bytes, void* stream) {
  if (mode != SP24_SCALE_DYNAMIC && mode != SP24_SCALE_STATIC) return SP24_ERR_MODE;
  if (!x_bf16 || !q_out || !scale_dev) return SP24_ERR_NULL;
  if (count < 1 || count > ((int64_t)1 << 40)) return SP24_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(q_out) || ((uintptr_t)scale_dev & 3u)) return SP24_ERR_ALIGN;
  const size_t need = mode == SP24_SCALE_DYNAMIC ? quant_workspace_bytes(count) : 0;
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return SP24_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return SP24_ERR_ALIGN;
  const size_t xb = (size_t)count * 2;
  if (overlaps(q_out, count, x_bf16, xb) || overlaps(scale_dev, 4, x_bf16, xb) ||
      overlaps(scale_dev, 4, q_out, count) ||
      (need > 0 && (overlaps(ws, need, x_bf16, xb) || overlaps(ws, need, q_out, count) ||
                    overlaps(ws, need, scale_dev, 4))))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_quant(dtype, static_cast<const uint16_t*>(x_bf16), count, q_out, scale_dev, mode,
                             need > 0 ? ws : nullptr, s),
                s);
}

int sp24_quant_fp8(const void* x_bf16, int64_t count, uint8_t* q_out, float* scale_dev, int mode,
                   void* ws, size_t ws_bytes, void* stream) {
  return quant_common(SP24_FP8_E4M3, x_bf16, count, q_out, scale_dev, mode, ws, ws_bytes, stream);
}

int sp24_quant_int8(const void* x_bf16, int64_t count, int8_t* q_out, float* scale_dev, int mode,
                    void* ws, size_t ws_bytes, void* stream) {
  return quant_common(SP24_INT8, x_bf16, count, reinterpret_cast<uint8_t*>(q_out), scale_dev, mode, ws,
                      ws_bytes, stream);
}

static int gemm_common(bool sparse, int dtype, int64_t m, int64_t n, int64_t k, const void* x,
                       const float* x_scale, const void* w, const uint32_t* meta,
                       const float* w_scale, void* y, void* ws, size_t ws_bytes, void* stream,
                       int xs_step = 0) {
  if (!known_dtype(dtype)) return SP24_ERR_DTYPE;
  if (!x || !w || !y || (sparse && !meta)) return SP24_ERR_NULL;
  if (scaled_dtype(dtype) && (!x_scale || !w_scale)) return SP24_ERR_NULL;
  sp24_plan p;
  int st = plan_gemm(sparse ? SP24_OP_GEMM : SP24_OP_DENSE_GEMM, dtype, m, n, k, &p);
  if (st != SP24_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (sparse && !aligned16(meta)))
    return SP24_ERR_ALIGN;
  if (scaled_dtype(dtype) && (((uintptr_t)x_scale & 3u) || ((uintptr_t)w_scale & 3u)))
    return SP24_ERR_ALIGN;
  if (p.workspace_bytes > 0) {
    if (ws == nullptr || ws_bytes < p.workspace_bytes) return SP24_ERR_WORKSPACE;
    if (!aligned16(ws)) return SP24_ERR_ALIGN;
  }
  const int es = esize(dtype);
  const size_t xb = (size_t)m * k * es, yb = (size_t)m * n * 2;
  const size_t wb = sparse ? (size_t)n * (k / 2) * es : (size_t)n * k * es;
  const size_t mb = sparse ? (size_t)n * (k / 32) * 4 : 0;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb) || (sparse && overlaps(y, yb, meta, mb)))
    return SP24_ERR_ALIAS;
  const size_t xsb = xs_step ? (size_t)m * 4 : 4;  // bytes of X scales: one per tensor or per row
  if (scaled_dtype(dtype) && (overlaps(y, yb, x_scale, xsb) || overlaps(y, yb, w_scale, 4)))
    return SP24_ERR_ALIAS;
  if (p.workspace_bytes > 0 &&
      (overlaps(ws, p.workspace_bytes, y, yb) || overlaps(ws, p.workspace_bytes, x, xb) ||
       overlaps(ws, p.workspace_bytes, w, wb)))
    return SP24_ERR_ALIAS;

  GemmArgs a;
  a.dtype = dtype;
  a.sparse = sparse;
  a.m = (int)m;
  a.n = (int)n;
  a.k = (int)k;
  a.x = x;
  a.x_scale = x_scale;
  a.w = w;
  a.meta = meta;
  a.w_scale = w_scale;
  a.y = static_cast<uint16_t*>(y);
  a.partial = p.split_k > 1 ? static_cast<float*>(ws) : nullptr;
  a.x_scale_step = xs_step;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_plan(a, p, s), s);
}

int sp24_gemm(int dtype, int64_t m, int64_t n, int64_t k, const void* x, const float* x_scale_dev,
              const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
              void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(true, dtype, m, n, k, x, x_scale_dev, w_values, w_meta, w_scale_dev, y_bf16, ws,
                     ws_bytes, stream);
}

int sp24_dense_gemm(int dtype, int64_t m, int64_t n, int64_t k, const void* x,
                    const float* x_scale_dev, const void* w_dense, const float* w_scale_dev,
                    void* y_bf16, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(false, dtype, m, n, k, x, x_scale_dev, w_dense, nullptr, w_scale_dev, y_bf16, ws,
                     ws_bytes, stream);
}

static int quant_rows_common(int dtype, const void* x_bf16, int64_t m, int64_t k, uint8_t* q_out,
                             float* scales_dev, void* stream) {
  if (!x_bf16 || !q_out || !scales_dev) return SP24_ERR_NULL;
  if (m < 1 || k < 8 || k % 8 != 0 || m > kMaxDim || k > kMaxDim || m * k > ((int64_t)1 << 40))
    return SP24_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(q_out) || ((uintptr_t)scales_dev & 3u)) return SP24_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, qb = (size_t)m * k, sb = (size_t)m * 4;
  if (overlaps(q_out, qb, x_bf16, xb) || overlaps(scales_dev, sb, x_bf16, xb) ||
      overlaps(scales_dev, sb, q_out, qb))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_quant_rows(dtype, static_cast<const uint16_t*>(x_bf16), m, k, q_out, scales_dev, s), s);
}

int sp24_quant_fp8_rows(const void* x_bf16, int64_t m, int64_t k, uint8_t* q_out, float* scales_dev,
                        void* stream) {
  return quant_rows_common(SP24_FP8_E4M3, x_bf16, m, k, q_out, scales_dev, stream);
}

int sp24_quant_int8_rows(const void* x_bf16, int64_t m, int64_t k, int8_t* q_out, float* scales_dev,
                         void* stream) {
  return quant_rows_common(SP24_INT8, x_bf16, m, k, reinterpret_cast<uint8_t*>(q_out), scales_dev, stream);
}

int sp24_slide_prune_pack(const void* w_bf16, int64_t n, int64_t k, int n_pat, void* w_out_bf16,
                          void* stream) {
  if (!w_bf16 || !w_out_bf16) return SP24_ERR_NULL;
  if (n_pat < 3 || n_pat > 8) return SP24_ERR_MODE;
  if (n < 1 || k < 2 * n_pat || k % (2 * n_pat) != 0 || n > kMaxDim || k > kMaxDim) return SP24_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(w_out_bf16)) return SP24_ERR_ALIGN;
  const int64_t kp = k / (2 * n_pat) * 4 * (n_pat - 1);
  if (overlaps(w_bf16, (size_t)n * k * 2, w_out_bf16, (size_t)n * kp * 2)) return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_slide_prune_pack(static_cast<const uint16_t*>(w_bf16), n, k, n_pat,
                                        static_cast<uint16_t*>(w_out_bf16), s),
                s);
}

namespace {
int slide_quant_common(int dtype, const void* x_bf16, int64_t m, int64_t k, int n_pat, uint8_t* q_out,
                       float* scales_dev, void* stream) {
  if (!x_bf16 || !q_out || !scales_dev) return SP24_ERR_NULL;
  if (n_pat < 3 || n_pat > 8) return SP24_ERR_MODE;
  if (m < 1 || k < 8 || k % 8 != 0 || k % (2 * n_pat) != 0 || m > kMaxDim || k > kMaxDim ||
      m * k > ((int64_t)1 << 40))
    return SP24_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(q_out) || ((uintptr_t)scales_dev & 3u)) return SP24_ERR_ALIGN;
  const int64_t kp = k / (2 * n_pat) * 4 * (n_pat - 1);
  const size_t xb = (size_t)m * k * 2, qb = (size_t)m * kp, sb = (size_t)m * 4;
  if (overlaps(q_out, qb, x_bf16, xb) || overlaps(scales_dev, sb, x_bf16, xb) ||
      overlaps(scales_dev, sb, q_out, qb))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(
      launch_slide_quant_rows(dtype, static_cast<const uint16_t*>(x_bf16), m, k, n_pat, q_out, scales_dev, s), s);
}
}  // namespace

int sp24_slide_quant_fp8_rows(const void* x_bf16, int64_t m, int64_t k, int n_pat, uint8_t* q_out,
                              float* scales_dev, void* stream) {
  return slide_quant_common(SP24_FP8_E4M3, x_bf16, m, k, n_pat, q_out, scales_dev, stream);
}

int sp24_slide_quant_int8_rows(const void* x_bf16, int64_t m, int64_t k, int n_pat, int8_t* q_out,
                               float* scales_dev, void* stream) {
  return slide_quant_common(SP24_INT8, x_bf16, m, k, n_pat, reinterpret_cast<uint8_t*>(q_out), scales_dev,
                            stream);
}

int sp24_gemm_rows(int dtype, int64_t m, int64_t n, int64_t k, const void* x, const float* x_scales_dev,
                   const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                   void* ws, size_t ws_bytes, void* stream) {
  if (!scaled_dtype(dtype)) return SP24_ERR_DTYPE;
  return gemm_common(true, dtype, m, n, k, x, x_scales_dev, w_values, w_meta, w_scale_dev, y_bf16,
                     ws, ws_bytes, stream, 1);
}

int sp24_gemm_qx(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scale_dev,
                 const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                 void* ws, size_t ws_bytes, void* stream) {
  return gemm_qx_common(m, n, k, x_bf16, x_scale_dev, w_values, w_meta, w_scale_dev, y_bf16, ws, ws_bytes,
                        false, stream);
}

int sp24_gemm_qx_noalloc(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scale_dev,
                         const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                         void* stream) {
  return gemm_qx_common(m, n, k, x_bf16, x_scale_dev, w_values, w_meta, w_scale_dev, y_bf16, nullptr, 0, true,
                        stream);
}

namespace {
// sp24_gemm_rows_qx (lift = 0, xk = k) and sp24_slide_gemm_qx (lift = N, X rows
// of xk values, the GEMM over k = K').
int rows_qx_common(int lift, int64_t m, int64_t n, int64_t k, int64_t xk, const void* x_bf16,
                   float* x_scales_dev, const void* w_values, const uint32_t* w_meta, const float* w_scale_dev,
                   void* y_bf16, void* ws, size_t ws_bytes, void* stream) {
  if (!x_bf16 || !x_scales_dev || !w_values || !w_meta || !w_scale_dev || !y_bf16) return SP24_ERR_NULL;
  sp24_plan p;
  int st = plan_qx(m, n, k, true, &p);
  if (st != SP24_OK) return st;
  if (!aligned16(x_bf16) || !aligned16(w_values) || !aligned16(w_meta) || !aligned16(y_bf16))
    return SP24_ERR_ALIGN;
  if (((uintptr_t)x_scales_dev & 3u) || ((uintptr_t)w_scale_dev & 3u)) return SP24_ERR_ALIGN;
  const QxWorkspace wsp = qx_workspace(p, m, k, true);
  if (wsp.total > 0) {
    if (ws == nullptr || ws_bytes < wsp.total) return SP24_ERR_WORKSPACE;
    if (!aligned16(ws)) return SP24_ERR_ALIGN;
  }
  const size_t xb = (size_t)m * xk * 2, yb = (size_t)m * n * 2, wb = (size_t)n * (k / 2);
  const size_t mb = (size_t)n * (k / 32) * 4, sb = (size_t)m * 4;
  const void* in[4] = {x_bf16, w_values, w_meta, w_scale_dev};
  const size_t inb[4] = {xb, wb, mb, 4};
  for (int i = 0; i < 4; ++i)
    if (overlaps(y_bf16, yb, in[i], inb[i]) || overlaps(x_scales_dev, sb, in[i], inb[i]) ||
        (wsp.total > 0 && overlaps(ws, wsp.total, in[i], inb[i])))
      return SP24_ERR_ALIAS;
  if (overlaps(y_bf16, yb, x_scales_dev, sb) ||
      (wsp.total > 0 && (overlaps(ws, wsp.total, y_bf16, yb) || overlaps(ws, wsp.total, x_scales_dev, sb))))
    return SP24_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  GemmArgs a;
  a.dtype = SP24_FP8_E4M3;
  a.sparse = true;
  a.m = (int)m;
  a.n = (int)n;
  a.k = (int)k;
  a.x_scale = x_scales_dev;  // one scale per row, also for the split-K reduction
  a.x_scale_step = 1;
  a.w = w_values;
  a.meta = w_meta;
  a.w_scale = w_scale_dev;
  a.y = static_cast<uint16_t*>(y_bf16);
  a.partial = p.split_k > 1 ? reinterpret_cast<float*>(wsb) : nullptr;
  if (wsp.fused) {
    a.x = nullptr;
    a.x_bf16 = static_cast<const uint16_t*>(x_bf16);
    a.x_scale_out = x_scales_dev;
    a.x_rows = true;
    a.x_lift = lift;
    return finish(launch_plan(a, p, s), s);
  }
  uint8_t* codes = wsb + wsp.gemm;
  hipError_t e = lift ? launch_slide_quant_rows(SP24_FP8_E4M3, static_cast<const uint16_t*>(x_bf16), m, xk, lift,
                                                codes, x_scales_dev, s)
                      : launch_quant_rows(SP24_FP8_E4M3, static_cast<const uint16_t*>(x_bf16), m, k, codes,
                                          x_scales_dev, s);
  a.x = codes;
  if (e == hipSuccess) e = launch_plan(a, p, s);
  return finish(e, s);
}
}  // namespace

int sp24_gemm_rows_qx(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scales_dev,
                      const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                      void* ws, size_t ws_bytes, void* stream) {
  return rows_qx_common(0, m, n, k, k, x_bf16, x_scales_dev, w_values, w_meta, w_scale_dev, y_bf16, ws, ws_bytes,
                        stream);
}

int sp24_slide_gemm_qx(int n_pat, int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scales_dev,
                       const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                       void* ws, size_t ws_bytes, void* stream) {
  if (n_pat < 3 || n_pat > 8) return SP24_ERR_MODE;
  if (k < 8 || k % 8 != 0 || k % (2 * n_pat) != 0 || k > kMaxDim) return SP24_ERR_SHAPE;
  const int64_t kp = k / (2 * n_pat) * 4 * (n_pat - 1);
  return rows_qx_common(n_pat, m, n, kp, k, x_bf16, x_scales_dev, w_values, w_meta, w_scale_dev, y_bf16, ws,
                        ws_bytes, stream);
}

int sp24_quant_fp8_groups(const void* x_bf16, int64_t rows, int64_t cols, int64_t group, uint8_t* q_out,
                          float* scales_dev, void* stream) {
  if (!x_bf16 || !q_out || !scales_dev) return SP24_ERR_NULL;
  if (rows < 1 || cols < 8 || group < 8 || group % 8 != 0 || cols % group != 0 || rows > kMaxDim || cols > kMaxDim ||
      rows * cols > ((int64_t)1 << 40))
    return SP24_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(q_out) || ((uintptr_t)scales_dev & 3u)) return SP24_ERR_ALIGN;
  const size_t xb = (size_t)rows * cols * 2, qb = (size_t)rows * cols, sb = (size_t)rows * (cols / group) * 4;
  if (overlaps(q_out, qb, x_bf16, xb) || overlaps(scales_dev, sb, x_bf16, xb) || overlaps(scales_dev, sb, q_out, qb))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_quant_groups(static_cast<const uint16_t*>(x_bf16), rows, cols, group, q_out, scales_dev, s), s);
}

int sp24_gemm_groups(int64_t m, int64_t n, int64_t k, int64_t group, const void* x, const float* x_scales_dev,
                     const void* w_values, const uint32_t* w_meta, const float* w_scales_dev, void* y_bf16, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!x || !x_scales_dev || !w_values || !w_meta || !w_scales_dev || !y_bf16) return SP24_ERR_NULL;
  if (group < 128 || group % 128 != 0 || k % group != 0) return SP24_ERR_SHAPE;
  const bool per_row = group == k;  // per-token X and per-output-channel W scales
  sp24_plan p;
  int st = per_row ? plan_gemm(SP24_OP_GEMM, SP24_FP8_E4M3, m, n, k, &p) : plan_groups(m, n, k, &p);
  if (st != SP24_OK) return st;
  const int64_t ng = k / group, gu = group / 128;
  if (!per_row) {  // K slices must hold whole groups (a finer plan than the 128-K one splits less)
    while (p.split_k > 1 && (k / 128 / p.split_k) % gu != 0) {
      p.split_k /= 2;
      p.grid_z = p.split_k;
    }
    if (p.split_k == 1) p.workspace_bytes = 0;
  }
  if (!aligned16(x) || !aligned16(w_values) || !aligned16(w_meta) || !aligned16(y_bf16)) return SP24_ERR_ALIGN;
  if (((uintptr_t)x_scales_dev & 3u) || ((uintptr_t)w_scales_dev & 3u)) return SP24_ERR_ALIGN;
  const size_t need = p.split_k > 1 ? (size_t)p.split_k * m * n * 4 : 0;
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return SP24_ERR_WORKSPACE;
    if (!aligned16(ws)) return SP24_ERR_ALIGN;
  }
  const size_t xb = (size_t)m * k, yb = (size_t)m * n * 2, wb = (size_t)n * (k / 2), mb = (size_t)n * (k / 32) * 4;
  const size_t xsb = (size_t)m * ng * 4, wsb = (size_t)n * ng * 4;
  const void* in[6] = {x, w_values, w_meta, x_scales_dev, w_scales_dev, nullptr};
  const size_t inb[6] = {xb, wb, mb, xsb, wsb, 0};
  for (int i = 0; i < 5; ++i)
    if (overlaps(y_bf16, yb, in[i], inb[i]) || (need > 0 && overlaps(ws, need, in[i], inb[i]))) return SP24_ERR_ALIAS;
  if (need > 0 && overlaps(ws, need, y_bf16, yb)) return SP24_ERR_ALIAS;

  GemmArgs a;
  a.dtype = SP24_FP8_E4M3;
  a.sparse = true;
  a.m = (int)m;
  a.n = (int)n;
  a.k = (int)k;
  a.x = x;
  a.w = w_values;
  a.meta = w_meta;
  a.y = static_cast<uint16_t*>(y_bf16);
  a.partial = p.split_k > 1 ? static_cast<float*>(ws) : nullptr;
  if (per_row) {
    a.x_scale = x_scales_dev;
    a.x_scale_step = 1;
    a.w_scale = w_scales_dev;
    a.w_scale_step = 1;
  } else {
    a.x_gscale = x_scales_dev;
    a.w_gscale = w_scales_dev;
    a.group_units = (int)gu;
    a.n_groups = (int)ng;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_plan(a, p, s), s);
}

int sp24_palette_analyze(const void* w_bf16, int64_t n, int64_t k, uint8_t* palette_dev, int32_t* row_slot_dev,
                         int32_t* counts_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!w_bf16 || !palette_dev || !row_slot_dev || !counts_dev) return SP24_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n > kMaxDim || k > kMaxDim || n > INT_MAX) return SP24_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(palette_dev) || ((uintptr_t)row_slot_dev & 3u) || ((uintptr_t)counts_dev & 3u))
    return SP24_ERR_ALIGN;
  const size_t need = palette_analyze_ws_bytes(n);
  if (ws == nullptr || ws_bytes < need) return SP24_ERR_WORKSPACE;
  if (!aligned16(ws)) return SP24_ERR_ALIGN;
  const size_t wb = (size_t)n * k * 2, sb = (size_t)n * 4;
  const void* outs[4] = {palette_dev, row_slot_dev, counts_dev, ws};
  const size_t outb[4] = {16, sb, 8, need};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(outs[i], outb[i], w_bf16, wb)) return SP24_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outb[i], outs[j], outb[j])) return SP24_ERR_ALIAS;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_palette_analyze(static_cast<const uint16_t*>(w_bf16), n, k, palette_dev, row_slot_dev,
                                       counts_dev, ws, s),
                s);
}

int sp24_palette_pack(const void* w_bf16, int64_t n, int64_t k, const uint8_t* palette_dev,
                      const int32_t* row_slot_dev, int64_t n_pal, int64_t n_verb, uint8_t* sm_out,
                      uint32_t* ix_out, int32_t* pal_rows_out, void* verb_out, int32_t* verb_rows_out,
                      void* stream) {
  if (!w_bf16 || !palette_dev || !row_slot_dev) return SP24_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n > kMaxDim || k > kMaxDim || n > INT_MAX) return SP24_ERR_SHAPE;
  if (n_pal < 0 || n_verb < 0 || n_pal + n_verb != n) return SP24_ERR_SHAPE;
  if (n_pal > 0 && (!sm_out || !ix_out || !pal_rows_out)) return SP24_ERR_NULL;
  if (n_verb > 0 && (!verb_out || !verb_rows_out)) return SP24_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(palette_dev) || ((uintptr_t)row_slot_dev & 3u)) return SP24_ERR_ALIGN;
  if (n_pal > 0 && (!aligned16(sm_out) || !aligned16(ix_out) || ((uintptr_t)pal_rows_out & 3u)))
    return SP24_ERR_ALIGN;
  if (n_verb > 0 && (!aligned16(verb_out) || ((uintptr_t)verb_rows_out & 3u))) return SP24_ERR_ALIGN;
  const void* ins[3] = {w_bf16, palette_dev, row_slot_dev};
  const size_t inb[3] = {(size_t)n * k * 2, 16, (size_t)n * 4};
  const void* outs[5] = {sm_out, ix_out, pal_rows_out, verb_out, verb_rows_out};
  const size_t outb[5] = {pad16(n_pal) * k, pad16(n_pal) * k / 2, (size_t)n_pal * 4, pad16(n_verb) * k * 2,
                          (size_t)n_verb * 4};
  for (int i = 0; i < 5; ++i) {
    if (outb[i] == 0) continue;
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], outb[i], ins[j], inb[j])) return SP24_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (outb[j] != 0 && overlaps(outs[i], outb[i], outs[j], outb[j])) return SP24_ERR_ALIAS;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_palette_pack(static_cast<const uint16_t*>(w_bf16), n, k, palette_dev, row_slot_dev, n_pal,
                                    n_verb, sm_out, ix_out, pal_rows_out, static_cast<uint16_t*>(verb_out),
                                    verb_rows_out, s),
                s);
}

int sp24_palette_decode(const sp24_palette_weight* pw, int64_t n, int64_t k, void* w_out_bf16, void* stream) {
  if (!w_out_bf16) return SP24_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n > kMaxDim || k > kMaxDim || n > INT_MAX) return SP24_ERR_SHAPE;
  const int st = check_palette(pw, n);
  if (st != SP24_OK) return st;
  if (!aligned16(w_out_bf16)) return SP24_ERR_ALIGN;
  if (overlaps_palette(w_out_bf16, (size_t)n * k * 2, pw, k)) return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_palette_decode(palette_args(pw), n, k, static_cast<uint16_t*>(w_out_bf16), s), s);
}

int sp24_palette_gemm(int64_t m, int64_t n, int64_t k, const void* x_bf16, const sp24_palette_weight* pw,
                      void* y_bf16, void* ws, size_t ws_bytes, void* stream) {
  if (!x_bf16 || !y_bf16) return SP24_ERR_NULL;
  const PaletteWs wsp = palette_gemm_ws(m, n, k);
  if (!wsp.ok || n > INT_MAX) return SP24_ERR_SHAPE;
  const int st = check_palette(pw, n);
  if (st != SP24_OK) return st;
  if (!aligned16(x_bf16) || !aligned16(y_bf16)) return SP24_ERR_ALIGN;
  if (wsp.total > 0) {
    if (ws == nullptr || ws_bytes < wsp.total) return SP24_ERR_WORKSPACE;
    if (!aligned16(ws)) return SP24_ERR_ALIGN;
  }
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 2;
  if (overlaps(y_bf16, yb, x_bf16, xb) || overlaps_palette(y_bf16, yb, pw, k)) return SP24_ERR_ALIAS;
  if (wsp.total > 0 && (overlaps(ws, wsp.total, x_bf16, xb) || overlaps(ws, wsp.total, y_bf16, yb) ||
                        overlaps_palette(ws, wsp.total, pw, k)))
    return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PaletteArgs pa = palette_args(pw);
  if (m <= kPaletteMaxM)
    return finish(launch_palette_gemm_small(static_cast<const uint16_t*>(x_bf16), pa, static_cast<uint16_t*>(y_bf16),
                                            (int)m, (int)n, (int)k, s),
                  s);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  uint16_t* wd = reinterpret_cast<uint16_t*>(wsb);
  hipError_t e = launch_palette_decode(pa, n, k, wd, s);
  if (e == hipSuccess) {
    GemmArgs a;
    a.dtype = SP24_BF16;
    a.sparse = false;
    a.m = (int)m;
    a.n = (int)n;
    a.k = (int)k;
    a.x = x_bf16;
    a.x_scale = nullptr;
    a.w = wd;
    a.meta = nullptr;
    a.w_scale = nullptr;
    a.y = static_cast<uint16_t*>(y_bf16);
    a.partial = wsp.plan.split_k > 1 ? reinterpret_cast<float*>(wsb + wsp.weight) : nullptr;
    e = launch_plan(a, wsp.plan, s);
  }
  return finish(e, s);
}

}  // extern "C"
