/*
 * sp24.h -- C ABI of libsp24: 2:4 structured-sparse GEMM Y = X . W^T for
 * gfx950 (AMD Instinct MI355X), BF16, FP8-E4M3 or INT8 operands, fp32
 * accumulation (exact int32 sums for INT8), BF16 output.
 *
 * Operation sources ("the cookbook" = the page "Deploying 2:4 Sparsity with
 * FP8 on Hopper: A Production Cookbook"):
 *   - 2:4 magnitude pruning: the cookbook, pipeline step 4 (keep the two
 *     largest-magnitude values of every group of 4) and step 2 (groups are 4
 *     contiguous values along the inner dimension K of the [out, in] weight);
 *     Practical Example 1 (top-2 of |w| per group of 4 along the chosen axis).
 *   - Compressed form: the SlideSparse page ("SlideSparse: Fast and Flexible
 *     (2N-2):2N Structured Sparsity") has weights converted once, offline, to
 *     the hardware's compressed layout; this library defines that layout below.
 *   - Per-tensor dynamic FP8 scaling with a clip at the format maximum: the
 *     cookbook, pipeline steps 3 and 6 and "Troubleshooting quick hits".
 *   - INT8 W8A8 beside 2:4 + FP8: the cookbook's table "Precision and sparsity
 *     recipes" and pipeline step 6 "INT8 alternative"; its symmetric scale
 *     amax/127 and round-half-even codes in [-127, 127] are this library's
 *     reading (no page fixes them).
 *   - The sparse product on the linear/FFN projections: the cookbook, pipeline
 *     step 2 and its "What to prune" table.
 *   - Lossless BF16 exponent-palette weights (sp24_palette_*): the page "Unweight:
 *     Compresion Lossless de Pesos de LLM para Inferencia en GPU H100",
 *     architecture (16-entry exponent palette, verbatim rows) and execution
 *     pipelines ("direct palette" and "full decode").
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, contiguous, row-major device buffers owned by the
 *     caller.  The library never allocates or frees device memory and keeps no
 *     mutable global state; calls are reentrant.  The one exception is
 *     sp24_gemm_qx_noalloc, whose scratch memory is a fixed array per GPU (see
 *     there).
 *   - W is [n, k] (the nn.Linear weight layout), X is [m, k], Y is [m, n].
 *   - bf16 buffers hold IEEE bfloat16 bit patterns; FP8 buffers hold OCP
 *     E4M3FN byte codes (bias 7, max 448, NaN = 0x7F/0xFF, no infinities);
 *     INT8 buffers hold two's-complement bytes (the quantisers write -127..127).
 *   - Compressed weight of W [n, k]:
 *       values [n, k/2]: the two kept values of group g (columns 4g..4g+3) at
 *                        columns 2g and 2g+1, in ascending position order;
 *       meta   n * k/32 uint32 words: word w of row r holds, at bits
 *                        4*(g % 8), the nibble (i0 | i1 << 2) of group
 *                        g = 8w + (g % 8), i0 < i1 the kept positions inside the
 *                        group.  Storage order: the k/32 words of a row are cut
 *                        into blocks of 4 (128 values of k); block b holds every
 *                        row's words of that block, row after row (a last block
 *                        of fewer than 4 words likewise), so word w of row r sits
 *                        at 4*n*(w/4) + r*min(4, k/32 - 4*(w/4)) + w%4.  A K step
 *                        of a row range is then contiguous.
 *     The kept pair of a group: the two largest |w|, magnitudes compared
 *     exactly, ties to the lower index, +0 == -0.  Inputs must be finite.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; results are visible after the stream is synchronised.
 *   - Every argument is validated before any HIP call.  The return value is
 *     SP24_OK or a negative sp24_status.  Faults inside a kernel surface at the
 *     caller's next synchronisation; with the environment variable
 *     SP24_SYNC_CHECK=1 every call synchronises its stream and reports them.
 *   - Device pointers must be 16-byte aligned.  Outputs must not overlap inputs.
 */
#ifndef SP24_H
#define SP24_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SP24_VERSION 100 /* 1.0.0 */

typedef enum sp24_status {
  SP24_OK = 0,
  SP24_ERR_NULL = -1,      /* a required pointer is NULL */
  SP24_ERR_SHAPE = -2,     /* a size is out of range (see each call) */
  SP24_ERR_ALIGN = -3,     /* a device pointer is not 16-byte aligned */
  SP24_ERR_DTYPE = -4,     /* unknown dtype */
  SP24_ERR_WORKSPACE = -5, /* workspace missing or smaller than sp24_workspace_size() */
  SP24_ERR_HIP = -6,       /* a HIP launch or (with SP24_SYNC_CHECK) a kernel failed */
  SP24_ERR_MODE = -7,      /* unknown scale mode or op */
  SP24_ERR_ALIAS = -8      /* an output overlaps an input */
} sp24_status;

typedef enum sp24_dtype {
  SP24_BF16 = 0,      /* bfloat16 operands, no scales */
  SP24_FP8_E4M3 = 1,  /* OCP E4M3FN codes with one fp32 scale per tensor */
  SP24_INT8 = 2       /* int8 codes with one fp32 scale per tensor; int32 sums */
} sp24_dtype;

typedef enum sp24_scale_mode {
  SP24_SCALE_DYNAMIC = 0, /* compute s = amax/448 (INT8: amax/127) on the device and store it */
  SP24_SCALE_STATIC = 1   /* use the scale already stored at scale_dev */
} sp24_scale_mode;

typedef enum sp24_op {
  SP24_OP_GEMM = 0,       /* sp24_gemm */
  SP24_OP_QUANT = 1,      /* sp24_quant_fp8, sp24_quant_int8 */
  SP24_OP_DENSE_GEMM = 2, /* sp24_dense_gemm */
  SP24_OP_GEMM_QX = 3,    /* sp24_gemm_qx (dtype SP24_FP8_E4M3) */
  SP24_OP_PALETTE_ANALYZE = 4, /* sp24_palette_analyze (n = rows, k; m and dtype ignored) */
  SP24_OP_PALETTE_GEMM = 5,    /* sp24_palette_gemm (dtype ignored) */
  SP24_OP_GEMM_ROWS_QX = 6,    /* sp24_gemm_rows_qx; sp24_slide_gemm_qx with k = K' (dtype SP24_FP8_E4M3) */
  SP24_OP_GEMM_GROUPS = 7      /* sp24_gemm_groups, any group (dtype SP24_FP8_E4M3) */
} sp24_op;

typedef enum sp24_kernel {
  SP24_KERNEL_SKINNY = 0, /* small m: operands straight to registers, K split across waves */
  SP24_KERNEL_TILED = 1,  /* large m: 256 x 256 tiles staged through an LDS ring */
  SP24_KERNEL_STREAM = 2  /* small m: one row range per workgroup, operands through an LDS ring */
} sp24_kernel;

/* Launch plan chosen by the host from (op, dtype, m, n, k).  Pure host logic:
 * sp24_plan() makes no HIP call, so it can be inspected without a GPU. */
typedef struct sp24_plan {
  int kernel;             /* sp24_kernel */
  int tile_n;             /* rows of W per workgroup (stream kernel: the rows of its range) */
  int tile_m;             /* rows of X per workgroup */
  int waves;              /* waves (64 lanes) per workgroup */
  int split_k;            /* number of K slices reduced through the workspace (1: none) */
  int grid_x, grid_y, grid_z;
  int config;             /* kernel configuration id inside the kernel family */
  int batch;              /* skinny: chunks of K whose loads are issued together;
                             stream: 128-K units per wave per step */
  size_t workspace_bytes; /* bytes of workspace this plan needs */
} sp24_plan;

/* Prune W [n, k] (bf16) to 2:4 along k and compress it.
 *   w_bf16      in : [n, k] bf16
 *   values_bf16 out: [n, k/2] bf16
 *   meta        out: n * k/32 uint32 words (storage order above)
 * Requires n >= 1, k >= 32, k % 32 == 0.  Dropped values are not stored. */
int sp24_prune_compress(const void* w_bf16, int64_t n, int64_t k, void* values_bf16,
                        uint32_t* meta, void* stream);

/* Rebuild the dense pruned W [n, k] from (values, meta): kept values at their
 * positions, all-zero bit patterns (+0) elsewhere.
 *   dtype  SP24_BF16 (values and w_out are bf16), SP24_FP8_E4M3 or SP24_INT8 (byte codes)
 * Requires n >= 1, k >= 32, k % 32 == 0.  Nibbles are used as given: a nibble
 * with i0 == i1 (never written by sp24_prune_compress) writes both values to
 * one position, the second last; every write stays inside the row. */
int sp24_decompress(int dtype, const void* values, const uint32_t* meta, int64_t n, int64_t k,
                    void* w_out, void* stream);

/* Count the metadata nibbles of a compressed weight that are not a valid kept
 * pair (i0 < i1, i.e. one of 4, 8, 9, 12, 13, 14): a check for compressed
 * weights that did not come from sp24_prune_compress (sp24_gemm and
 * sp24_decompress use nibbles as given).
 *   meta    in : n * k/32 uint32 words (storage order above)
 *   bad_dev out: one uint32 on the device; the count is ADDED to it (the
 *                caller zeroes it first), so several tensors can share one.
 * Requires n >= 1, k >= 32, k % 32 == 0; bad_dev 4-byte aligned. */
int sp24_check_meta(const uint32_t* meta, int64_t n, int64_t k, uint32_t* bad_dev, void* stream);

/* Quantise count bf16 values to E4M3 codes with one per-tensor scale.
 *   mode SP24_SCALE_DYNAMIC: amax = max|x| over the tensor (exact), then
 *        *scale_dev = fp32(amax / 448) (1.0 if amax == 0), written by the
 *        device (no host synchronisation); needs a workspace.
 *   mode SP24_SCALE_STATIC : *scale_dev is read, not written; no workspace.
 *   Each value: q = e4m3_rne(clamp(fp32(x / s), -448, 448)) with the IEEE
 *   float32 quotient (values beyond the range saturate to +-448); with a dynamic
 *   scale and amax >= 2^-63 the kernels form it as x * fp32(1/s) plus one
 *   exact-residual correction, which gives the same code for every bf16 x.
 *   x_bf16 in: [count] bf16; q_out out: [count] bytes; scale_dev: one fp32 on
 *   the device.  count >= 1.  ws/ws_bytes: sp24_workspace_size(SP24_OP_QUANT, ...). */
int sp24_quant_fp8(const void* x_bf16, int64_t count, uint8_t* q_out, float* scale_dev, int mode,
                   void* ws, size_t ws_bytes, void* stream);

/* Quantise count bf16 values to INT8 codes with one per-tensor symmetric scale
 * (the cookbook's INT8 W8A8 recipe, table "Precision and sparsity recipes").
 * As sp24_quant_fp8 with the INT8 range:
 *   mode SP24_SCALE_DYNAMIC: *scale_dev = fp32(amax / 127) (1.0 if amax == 0).
 *   Each value: q = clamp(round_half_even(fp32(x / s)), -127, 127) with an IEEE
 *   float32 division (-128 is never written).  Inputs must be finite.
 *   Workspace, limits and errors as sp24_quant_fp8 (op SP24_OP_QUANT). */
int sp24_quant_int8(const void* x_bf16, int64_t count, int8_t* q_out, float* scale_dev, int mode,
                    void* ws, size_t ws_bytes, void* stream);

/* Y = X . W^T with W in compressed 2:4 form; fp32 accumulation; bf16 output.
 *   dtype SP24_BF16    : x is bf16 [m, k], w_values bf16 [n, k/2]; scales ignored (may be NULL).
 *   dtype SP24_FP8_E4M3: x is E4M3 [m, k] with *x_scale_dev, w_values E4M3 [n, k/2]
 *                        with *w_scale_dev; y = bf16_rne(acc * fp32(sx * sw)).
 *   dtype SP24_INT8    : x int8 [m, k] with *x_scale_dev, w_values int8 [n, k/2] with
 *                        *w_scale_dev; the products are summed exactly in int32 (per
 *                        K slice when K is split), converted to fp32, then scaled as
 *                        FP8.  Also requires k <= 131072: a sum then stays below
 *                        2^31 in magnitude (at most k/2 products of at most
 *                        128 * 128 for any codes; the dense baseline's k products
 *                        of codes within [-127, 127], as the quantisers write).
 *   w_meta n * k/32 words (storage order above); y_bf16 [m, n].
 * Requires m >= 1, n >= 1, k >= 128, k % 128 == 0.  The sum over k is formed in
 * a fixed order for a given (m, n, k): results are bitwise reproducible.
 * ws/ws_bytes: at least sp24_workspace_size(SP24_OP_GEMM, dtype, m, n, k)
 * (may be NULL/0 when that is 0).  Every supported shape runs the sparse
 * kernels; there is no dense fallback. */
int sp24_gemm(int dtype, int64_t m, int64_t n, int64_t k, const void* x, const float* x_scale_dev,
              const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
              void* ws, size_t ws_bytes, void* stream);

/* Dense baseline for comparison: Y = X . W^T with an uncompressed W [n, k]
 * (bf16, E4M3 or INT8 codes) on dense MFMA; same scales, epilogue and limits as
 * sp24_gemm. */
int sp24_dense_gemm(int dtype, int64_t m, int64_t n, int64_t k, const void* x,
                    const float* x_scale_dev, const void* w_dense, const float* w_scale_dev,
                    void* y_bf16, void* ws, size_t ws_bytes, void* stream);

/* Per-token (per-row) E4M3 quantisation of X [m, k] (bf16): row r gets its own
 * dynamic scale scales_dev[r] = fp32(amax(|x[r, :]|) / 448) (1 for an all-zero
 * row) and its codes exactly as sp24_quant_fp8 would quantise that row alone.
 * The per-token quantisation of the SlideSparse page ("SlideSparse: Fast and
 * Flexible (2N-2):2N Structured Sparsity", activation lifting); finer scales
 * keep an outlier token from coarsening every other token's codes.
 *   x_bf16 in : [m, k] bf16, k % 8 == 0;  q_out out: [m, k] E4M3 codes;
 *   scales_dev out: [m] fp32.  No workspace, no host synchronisation. */
int sp24_quant_fp8_rows(const void* x_bf16, int64_t m, int64_t k, uint8_t* q_out, float* scales_dev,
                        void* stream);

/* Per-token INT8 quantisation: as sp24_quant_fp8_rows with the INT8 codes and
 * scale of sp24_quant_int8 (scales_dev[r] = fp32(amax_r / 127), 1 for a zero
 * row); row r is quantised exactly as sp24_quant_int8 would quantise it alone. */
int sp24_quant_int8_rows(const void* x_bf16, int64_t m, int64_t k, int8_t* q_out, float* scales_dev,
                         void* stream);

/* SlideSparse ("SlideSparse: Fast and Flexible (2N-2):2N Structured Sparsity",
 * technical summary, section 2): a (2N-2):2N weight on the 2:4 path.
 *
 * sp24_slide_prune_pack: prune W [n, k] (bf16) to (2N-2):2N along k (the 2N-2
 * largest magnitudes of every block of 2N, ties to the lower index) and write
 * the expanded weight W' [n, k'] (bf16), k' = k (2N-2)/N: block b becomes N-1
 * groups of 4, group j holding the values of window j (block positions 2j ..
 * 2j+3) that it owns, zeros elsewhere.  Window j owns the nonzero values at
 * positions 2j, 2j+1, then fills up to two from positions 2j+2, 2j+3 (the last
 * window owns whatever remains).  W' is 2:4 along k', so sp24_prune_compress
 * of W' keeps every value; multiply it with X' from sp24_slide_quant_fp8_rows.
 *   n_pat = N in [3, 8] (6:8 is N = 4); k % (2N) == 0.  Errors: SP24_ERR_MODE
 *   for N, the usual ones otherwise. */
int sp24_slide_prune_pack(const void* w_bf16, int64_t n, int64_t k, int n_pat, void* w_out_bf16,
                          void* stream);

/* Activation lifting fused into per-token quantisation: X [m, k] (bf16) ->
 * E4M3 codes of X' [m, k'] with X'[r, b*4(N-1) + 4j + p] = X[r, b*2N + 2j + p],
 * and scales_dev[r] = fp32(amax(|x[r, :]|) / 448) as sp24_quant_fp8_rows (the
 * lifted row has the same maximum), so X' . W'^T = X . W^T.
 *   k % 8 == 0 and k % (2N) == 0; q_out [m, k']; scales_dev [m]. */
int sp24_slide_quant_fp8_rows(const void* x_bf16, int64_t m, int64_t k, int n_pat, uint8_t* q_out,
                              float* scales_dev, void* stream);

/* The same lifting fused into per-token INT8 quantisation (the page's results
 * are INT8 W8A8): the codes and scales_dev[r] = fp32(amax_r / 127) of
 * sp24_quant_int8_rows, in the lifted order of sp24_slide_quant_fp8_rows.
 * Multiply with sp24_gemm_rows(SP24_INT8, ...) on INT8 weights of W'.
 *   Shapes, alignment and errors as sp24_slide_quant_fp8_rows. */
int sp24_slide_quant_int8_rows(const void* x_bf16, int64_t m, int64_t k, int n_pat, int8_t* q_out,
                               float* scales_dev, void* stream);

/* Y = X . W^T as sp24_gemm with dtype SP24_FP8_E4M3 or SP24_INT8, except that
 * X carries one scale per row: y[r, :] = bf16_rne(acc[r, :] * fp32(x_scales_dev[r] * sw)).
 *   x [m, k] codes (from sp24_quant_fp8_rows / sp24_quant_int8_rows);
 *   x_scales_dev [m] fp32; the rest, the workspace (sp24_workspace_size(
 *   SP24_OP_GEMM, dtype, ...)) and the errors as for sp24_gemm; SP24_BF16 is
 *   SP24_ERR_DTYPE. */
int sp24_gemm_rows(int dtype, int64_t m, int64_t n, int64_t k, const void* x, const float* x_scales_dev,
                   const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                   void* ws, size_t ws_bytes, void* stream);

/* Y = X . W^T for a bf16 X with FP8 weights: exactly sp24_quant_fp8(x_bf16,
 * m*k, codes, x_scale_dev, SP24_SCALE_DYNAMIC) followed by sp24_gemm(
 * SP24_FP8_E4M3, ..., codes, x_scale_dev, ...), bit for bit in y and in
 * *x_scale_dev, in one call.  The per-tensor scale follows the cookbook's
 * dynamic FP8 scaling ("Deploying 2:4 Sparsity with FP8 on Hopper", pipeline
 * step 3); the quantisation happens inside the GEMM kernel when X is small
 * (m*k <= 65536 values, the plan's small-m kernel has room for its tokens'
 * codes in LDS and each of its workgroups casts at most 16384 values: every
 * workgroup repeats the cast of its tokens), which saves the quantiser's launch
 * and the round trip of the codes through memory; otherwise the two steps run
 * as two launches with the codes in the workspace.
 *   x_bf16      in : [m, k] bf16
 *   x_scale_dev out: fp32, the scale amax(|x|)/448 (1 when x is all zero)
 *   w_values    in : [n, k/2] E4M3 codes; w_meta as for sp24_gemm;
 *   w_scale_dev in : fp32;  y_bf16 out: [m, n]
 * ws/ws_bytes: at least sp24_workspace_size(SP24_OP_GEMM_QX, SP24_FP8_E4M3, m,
 * n, k).  Same shape limits, alignment (x_scale_dev and w_scale_dev: 4 bytes)
 * and errors as sp24_gemm; x_scale_dev may alias no other argument. */
int sp24_gemm_qx(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scale_dev,
                 const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                 void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Finer FP8 scales: per output channel of W and per group of K.  The research-
 * roadmap page ("La Densite Dynamique et les Noyaux Non Structures ...",
 * quantisation under extreme sparsity) recommends per-channel or per-group
 * scales for outlier-heavy layers; this library's reading of them:
 *   - a group is `group` consecutive values of one row, quantised exactly as
 *     sp24_quant_fp8 would quantise those values alone (dynamic scale
 *     fp32(amax / 448), 1 for an all-zero group);
 *   - X [m, k] is quantised in groups along k; W in groups of its compressed
 *     values [n, k/2], group/2 of them for a group of k (the kept values of k
 *     positions [group*g, group*(g+1)) are compressed columns [group/2*g,
 *     group/2*(g+1)));
 *   - group == k is per-token X and per-output-channel W scales.
 * ------------------------------------------------------------------------- */

/* E4M3 codes of a bf16 [rows, cols] with one dynamic scale per group of `group`
 * consecutive values of a row.
 *   x_bf16 in : [rows, cols] bf16;  q_out out: [rows, cols] E4M3 codes;
 *   scales_dev out: [rows, cols/group] fp32, scale of group g of row r at
 *   scales_dev[r * (cols/group) + g].
 *   group % 8 == 0, cols % group == 0.  No workspace, no host synchronisation. */
int sp24_quant_fp8_groups(const void* x_bf16, int64_t rows, int64_t cols, int64_t group, uint8_t* q_out,
                          float* scales_dev, void* stream);

/* Y = X . W^T with FP8 codes carrying one scale per group of `group` values of k:
 *   y[r, c] = bf16_rne( sum over groups g of P_g * fp32(x_scales[r, g] * w_scales[c, g]) ),
 *   P_g the fp32 sum of the products of group g (k in [group*g, group*(g+1))).
 *   x [m, k] E4M3 codes, x_scales_dev [m, k/group]; w_values [n, k/2] E4M3 codes of
 *   the compressed weight quantised in groups of group/2 (sp24_quant_fp8_groups),
 *   w_scales_dev [n, k/group]; w_meta as for sp24_gemm; y_bf16 [m, n].
 *   group % 128 == 0 and k % group == 0.  group == k (per-token X, per-output-channel
 *   W) runs the plan of sp24_gemm with the two scale vectors applied in the
 *   epilogue; smaller groups run the small-m stream kernel at every m, which
 *   keeps the scales of its rows, tokens and K slice in LDS and scales each 128-K
 *   unit's partial product (the large-m kernel has no room for a second set of
 *   accumulators, so prefill shapes with groups are slower than with one scale
 *   per row).
 * ws/ws_bytes: at least sp24_workspace_size(SP24_OP_GEMM_GROUPS, SP24_FP8_E4M3, m,
 * n, k) (the same for every group).  Shape limits, alignment (scales: 4 bytes) and
 * errors as sp24_gemm. */
int sp24_gemm_groups(int64_t m, int64_t n, int64_t k, int64_t group, const void* x, const float* x_scales_dev,
                     const void* w_values, const uint32_t* w_meta, const float* w_scales_dev, void* y_bf16,
                     void* ws, size_t ws_bytes, void* stream);

/* Bytes of the scratch array that sp24_gemm_qx_noalloc keeps on each GPU. */
#define SP24_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* sp24_gemm_qx without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The result is bit for bit that of sp24_gemm_qx with
 * the same arguments (the same kernels run).  The workspace sp24_gemm_qx would
 * need (split-K partial sums, the E4M3 codes of X when they go through memory,
 * the quantiser's partial maxima) lives instead in one static array of
 * SP24_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on holds
 * from the first kernel launch until the process ends.  The call allocates and
 * frees nothing, and nothing in the array has to start at zero: every byte a
 * call reads there it wrote first.
 *   Arguments, layouts, shape limits, alignment and errors as sp24_gemm_qx,
 *   minus ws/ws_bytes.  SP24_ERR_WORKSPACE when sp24_workspace_size(
 *   SP24_OP_GEMM_QX, SP24_FP8_E4M3, m, n, k) exceeds SP24_NOALLOC_SCRATCH_BYTES
 *   (decode shapes fit; an 8192-token prefill does not).  The stream must belong
 *   to the current device: the array used is the current device's.
 *   The first call on a device looks the array's address up (a HIP runtime
 *   query; make that first call outside graph capture) and keeps it.
 *   Every call on one GPU shares that GPU's array: calls that may run at the
 *   same time on one GPU (different streams, or threads without ordering) race
 *   on it and give wrong results; calls ordered on one stream are safe. */
int sp24_gemm_qx_noalloc(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scale_dev,
                         const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                         void* stream);

/* Per-token FP8 quantisation fused into the sparse GEMM (the step left of the
 * GEMM that the SlideSparse page fuses into its per-token quantisation, and
 * the cookbook's FP8 activation step with one scale per token): exactly
 * sp24_quant_fp8_rows(x_bf16, m, k, codes, x_scales_dev) followed by
 * sp24_gemm_rows(SP24_FP8_E4M3, ..., codes, x_scales_dev, ...), bit for bit in
 * y and in x_scales_dev, in one call.  When the plan's small-m kernel has room
 * for its tokens' codes in LDS (decode shapes) each workgroup quantises its
 * own tokens, so no codes go through memory and no quantiser is launched;
 * otherwise the two steps run as two launches with the codes in the workspace.
 *   x_bf16 in : [m, k] bf16;  x_scales_dev out: [m] fp32, amax_r/448 (1 for a
 *   zero row);  w_values, w_meta, w_scale_dev, y_bf16 as for sp24_gemm_qx.
 * ws/ws_bytes: at least sp24_workspace_size(SP24_OP_GEMM_ROWS_QX,
 * SP24_FP8_E4M3, m, n, k).  Shape limits, alignment and errors as
 * sp24_gemm_qx; x_scales_dev may alias no other argument. */
int sp24_gemm_rows_qx(int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scales_dev,
                      const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                      void* ws, size_t ws_bytes, void* stream);

/* SlideSparse's per-call path in one call ("SlideSparse: Fast and Flexible
 * (2N-2):2N Structured Sparsity", technical summary, section 2): exactly
 * sp24_slide_quant_fp8_rows(x_bf16, m, k, n_pat, codes, x_scales_dev)
 * followed by sp24_gemm_rows(SP24_FP8_E4M3, m, n, k', codes, ...), bit for
 * bit, with k' = k (2N-2)/N and the weight W' of sp24_slide_prune_pack,
 * compressed and quantised.  At decode shapes the lifting and the per-token
 * quantisation both happen inside the GEMM kernel, as for sp24_gemm_rows_qx.
 *   x_bf16 [m, k]; w_values [n, k'/2]; w_meta [n, k'/32]; y_bf16 [m, n].
 *   n_pat = N in [3, 8] (SP24_ERR_MODE otherwise); k % 8 == 0 and
 *   k % (2N) == 0; k' must meet sp24_gemm's limits.
 * ws/ws_bytes: at least sp24_workspace_size(SP24_OP_GEMM_ROWS_QX,
 * SP24_FP8_E4M3, m, n, k').  Errors otherwise as sp24_gemm_rows_qx. */
int sp24_slide_gemm_qx(int n_pat, int64_t m, int64_t n, int64_t k, const void* x_bf16, float* x_scales_dev,
                       const void* w_values, const uint32_t* w_meta, const float* w_scale_dev, void* y_bf16,
                       void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Lossless BF16 exponent-palette weights (no sparsity).  The 8 exponent bits of
 * BF16 weights are highly redundant; sign and mantissa stay as one byte.  One
 * palette per tensor holds its 16 most common exponents (by count, ties to the
 * smaller exponent; unused entries 0xFF).  A row whose exponents are all in the
 * palette is stored as sign+mantissa bytes sm [k] (sign << 7 | mantissa) and
 * 4-bit palette indices ix [k/8] words (element 8g + t, t < 4, at bits
 * [8t, 8t+4) of word g; element 8g + 4 + t at bits [8t+4, 8t+8)); every other
 * row is stored verbatim (bf16).  Both kinds are compact, in ascending row
 * order, with their row numbers.  Encoding is exact: sp24_palette_decode gives
 * back W bit for bit.  Inputs must be finite; k % 128 == 0.
 *   Storage order of sm, ix and verb: the rows of each kind in blocks of 16
 *   (row count padded to a multiple of 16; padding is read, never stored), K in
 *   chunks of 512 (the last chunk T*128 values, T = 1..3, when k % 512 != 0).
 *   Inside a (block, chunk) tile the 16-byte pieces are ordered [piece j][lane
 *   group q][row r16]: lane group q holds K [32Tq, 32T(q+1)) of the chunk and
 *   piece j its j-th 16 bytes, so one 64-lane load reads 1 KB of consecutive
 *   memory.  Sizes: sm pad16(n_pal)*k bytes, ix pad16(n_pal)*k/8 words, verb
 *   pad16(n_verb)*k bf16.
 * ------------------------------------------------------------------------- */
typedef struct sp24_palette_weight {
  const uint8_t* palette;   /* device, 16 bytes, 16-byte aligned */
  int64_t n_pal;            /* rows in palette form */
  const uint8_t* sm;        /* device, pad16(n_pal)*k bytes (16-byte aligned; NULL if n_pal == 0) */
  const uint32_t* ix;       /* device, pad16(n_pal)*k/8 words (16-byte aligned; NULL if n_pal == 0) */
  const int32_t* pal_rows;  /* device [n_pal] row numbers, ascending (4-byte aligned) */
  int64_t n_verb;           /* rows stored verbatim; n_pal + n_verb == n */
  const void* verb;         /* device, pad16(n_verb)*k bf16 (16-byte aligned; NULL if n_verb == 0) */
  const int32_t* verb_rows; /* device [n_verb] row numbers, ascending (4-byte aligned) */
} sp24_palette_weight;

/* Encoding, first call: the palette and every row's slot.
 *   w_bf16       in : [n, k] bf16, k % 128 == 0
 *   palette_dev  out: 16 bytes (16-byte aligned)
 *   row_slot_dev out: [n] int32: slot p >= 0 of a paletted row, -(v + 1) of a verbatim row
 *   counts_dev   out: int32[2] = {n_pal, n_verb}, read by the caller to size the outputs
 *   ws/ws_bytes: sp24_workspace_size(SP24_OP_PALETTE_ANALYZE, 0, 0, n, k). */
int sp24_palette_analyze(const void* w_bf16, int64_t n, int64_t k, uint8_t* palette_dev, int32_t* row_slot_dev,
                         int32_t* counts_dev, void* ws, size_t ws_bytes, void* stream);

/* Encoding, second call: write the rows into their slots (from sp24_palette_analyze
 * of the same w).  n_pal + n_verb must equal n; a slot outside [0, n_pal) or
 * [0, n_verb) is skipped, never written.  Outputs as in sp24_palette_weight. */
int sp24_palette_pack(const void* w_bf16, int64_t n, int64_t k, const uint8_t* palette_dev,
                      const int32_t* row_slot_dev, int64_t n_pal, int64_t n_verb, uint8_t* sm_out,
                      uint32_t* ix_out, int32_t* pal_rows_out, void* verb_out, int32_t* verb_rows_out,
                      void* stream);

/* Rebuild W [n, k] (bf16) from its encoded form, bit for bit.  Row numbers
 * outside [0, n) are skipped. */
int sp24_palette_decode(const sp24_palette_weight* pw, int64_t n, int64_t k, void* w_out_bf16, void* stream);

/* Y = X . W^T (bf16 in, fp32 accumulation, bf16 out) with W in palette form.
 *   m <= 16: the "direct palette" pipeline: the encoded rows stream from memory
 *            and BF16 is rebuilt in registers right before the matrix
 *            instructions; no workspace.
 *   m > 16 : the "full decode" pipeline: W is rebuilt into the workspace, then
 *            the dense BF16 GEMM (sp24_dense_gemm) runs on it.
 *   x_bf16 [m, k]; y_bf16 [m, n]; k % 128 == 0; ws/ws_bytes:
 *   sp24_workspace_size(SP24_OP_PALETTE_GEMM, 0, m, n, k). */
int sp24_palette_gemm(int64_t m, int64_t n, int64_t k, const void* x_bf16, const sp24_palette_weight* pw,
                      void* y_bf16, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by an op at a shape (0 if none; also 0 for invalid
 * arguments, which the op itself then rejects). */
size_t sp24_workspace_size(int op, int dtype, int64_t m, int64_t n, int64_t k);

/* The launch plan sp24_gemm / sp24_dense_gemm would use (op SP24_OP_GEMM or
 * SP24_OP_DENSE_GEMM).  Host-only.  Returns SP24_OK or the error the op would
 * return for these sizes. */
int sp24_plan_gemm(int op, int dtype, int64_t m, int64_t n, int64_t k, sp24_plan* out);

/* Human-readable text of a status code (static storage). */
const char* sp24_status_string(int status);

/* SP24_VERSION of the built library. */
int sp24_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SP24_H */
