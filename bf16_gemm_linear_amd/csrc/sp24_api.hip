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
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

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

// SP24_TILE="config,split_k" overrides the small-m plan (tuning only; split_k 0
// keeps the automatic choice).
bool tile_override(int* cfg, int* sk) {
  const char* v = getenv("SP24_TILE");
  if (v == nullptr || v[0] == '\0') return false;
  int a, b;
  if (sscanf(v, "%d,%d", &a, &b) != 2) return false;
  if (a < 0 || (a >= kSkinnyConfigs && a != kTiledConfig) || b < 0 || b > 64) return false;
  *cfg = a;
  *sk = b;
  return true;
}

struct Cfg {
  int rb, mb, nw, batch;
};

Cfg skinny_cfg(int id) {
  switch (id) {
#define SP24_CFG_CASE(ID, RB, MB, NW, BATCH) \
  case ID: return Cfg{RB, MB, NW, BATCH};
    SP24_SKINNY_CONFIGS(SP24_CFG_CASE)
#undef SP24_CFG_CASE
  }
  return Cfg{1, 1, 8, 1};
}

}  // namespace

int plan_gemm(int op, int dtype, int64_t m, int64_t n, int64_t k, sp24_plan* out) {
  if (out == nullptr) return SP24_ERR_NULL;
  memset(out, 0, sizeof(*out));
  if (op != SP24_OP_GEMM && op != SP24_OP_DENSE_GEMM) return SP24_ERR_MODE;
  if (dtype != SP24_BF16 && dtype != SP24_FP8_E4M3) return SP24_ERR_DTYPE;
  if (m < 1 || n < 1 || k < 128 || k % 128 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim)
    return SP24_ERR_SHAPE;

  // Large m with enough 256 x 256 tiles to fill the chip: LDS-tiled kernel.
  const int64_t tiles = ((n + 255) / 256) * ((m + 255) / 256);
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
  int oid, osk;
  const bool forced = tile_override(&oid, &osk);
  if (forced) {
    id = oid;
    sk = osk;
  }
  if ((!forced && m > 256 && tiles >= 128) || (forced && id == kTiledConfig)) {
    if (tiles > INT_MAX) return SP24_ERR_SHAPE;
    out->kernel = SP24_KERNEL_TILED;
    out->tile_n = 256;
    out->tile_m = 256;
    out->waves = 8;
    out->split_k = 1;
    out->grid_x = (int)tiles;
    out->grid_y = 1;
    out->grid_z = 1;
    out->config = kTiledConfig;
    out->batch = 1;
    out->workspace_bytes = 0;
    return SP24_OK;
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
  sp24_plan p;
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
  if (dtype != SP24_BF16 && dtype != SP24_FP8_E4M3) return SP24_ERR_DTYPE;
  if (!values || !meta || !w_out) return SP24_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0 || n > kMaxDim || k > kMaxDim) return SP24_ERR_SHAPE;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(w_out)) return SP24_ERR_ALIGN;
  const size_t ob = (size_t)n * k * esize(dtype), vb = ob / 2, mb = (size_t)n * (k / 32) * 4;
  if (overlaps(w_out, ob, values, vb) || overlaps(w_out, ob, meta, mb)) return SP24_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_decompress(dtype, values, meta, n, k, w_out, s), s);
}

int sp24_quant_fp8(const void* x_bf16, int64_t count, uint8_t* q_out, float* scale_dev, int mode,
                   void* ws, size_t ws_bytes, void* stream) {
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
  return finish(launch_quant_fp8(static_cast<const uint16_t*>(x_bf16), count, q_out, scale_dev, mode,
                                 need > 0 ? ws : nullptr, s),
                s);
}

static int gemm_common(bool sparse, int dtype, int64_t m, int64_t n, int64_t k, const void* x,
                       const float* x_scale, const void* w, const uint32_t* meta,
                       const float* w_scale, void* y, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != SP24_BF16 && dtype != SP24_FP8_E4M3) return SP24_ERR_DTYPE;
  if (!x || !w || !y || (sparse && !meta)) return SP24_ERR_NULL;
  if (dtype == SP24_FP8_E4M3 && (!x_scale || !w_scale)) return SP24_ERR_NULL;
  sp24_plan p;
  int st = plan_gemm(sparse ? SP24_OP_GEMM : SP24_OP_DENSE_GEMM, dtype, m, n, k, &p);
  if (st != SP24_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (sparse && !aligned16(meta)))
    return SP24_ERR_ALIGN;
  if (dtype == SP24_FP8_E4M3 && (((uintptr_t)x_scale & 3u) || ((uintptr_t)w_scale & 3u)))
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
  if (dtype == SP24_FP8_E4M3 && (overlaps(y, yb, x_scale, 4) || overlaps(y, yb, w_scale, 4)))
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = p.kernel == SP24_KERNEL_TILED ? launch_gemm_tiled(a, p, s) : launch_gemm_skinny(a, p, s);
  if (e == hipSuccess && p.split_k > 1) e = launch_splitk_reduce(a, p.split_k, s);
  return finish(e, s);
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

}  // extern "C"
