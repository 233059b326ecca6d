/*
 * sp24_probe.h -- measurement and layout probes shipped in libsp24.
 *
 * These calls are not part of the GEMM path.  They pin down facts of gfx950
 * that the sparse kernels rely on and that the pages (written for other
 * hardware) cannot give: how the sparse matrix-core instructions (SMFMAC) map
 * lanes and index bits to matrix elements, their issue rate, and the HBM
 * streaming rate.  Same conventions as sp24.h: caller-owned device buffers,
 * asynchronous on `stream`, validation before any HIP call, SP24_* status.
 */
#ifndef SP24_PROBE_H
#define SP24_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction variants understood by the probes. */
typedef enum sp24_probe_variant {
  SP24_PROBE_SMFMAC_16x16x128_FP8 = 0,  /* v_smfmac_f32_16x16x128_fp8_fp8 */
  SP24_PROBE_SMFMAC_16x16x64_BF16_ABID0 = 1, /* v_smfmac_f32_16x16x64_bf16, abid 0 */
  SP24_PROBE_SMFMAC_16x16x64_BF16_ABID1 = 2, /* same, abid 1 */
  SP24_PROBE_SMFMAC_32x32x64_FP8 = 3,   /* v_smfmac_f32_32x32x64_fp8_fp8 */
  SP24_PROBE_SMFMAC_32x32x32_BF16_ABID0 = 4,
  SP24_PROBE_SMFMAC_32x32x32_BF16_ABID1 = 5,
  SP24_PROBE_MFMA_16x16x128_FP8 = 6,    /* dense v_mfma_f32_16x16x128_f8f6f4 (fp8 x fp8) */
  SP24_PROBE_MFMA_16x16x32_BF16 = 7,    /* dense v_mfma_f32_16x16x32_bf16 */
  SP24_PROBE_SMFMAC_16x16x128_I8 = 8,   /* v_smfmac_i32_16x16x128_i8 */
  SP24_PROBE_SMFMAC_32x32x64_I8 = 9,    /* v_smfmac_i32_32x32x64_i8 */
  SP24_PROBE_MFMA_16x16x64_I8 = 10,     /* dense v_mfma_i32_16x16x64_i8 */
  SP24_PROBE_MFMA_32x32x32_I8 = 11,     /* dense v_mfma_i32_32x32x32_i8 */
  SP24_PROBE_N_VARIANTS = 12
} sp24_probe_variant;

/* Run one instruction per experiment, accumulator starting at 0.
 * Experiment e uses one wave (64 lanes).  Per lane, with fixed strides:
 *   a   : 32 bytes at a   + (e*64 + lane)*32  (the A operand; 16 bytes used by
 *         sparse variants and by the dense bf16 and int8 variants, 32 by dense fp8)
 *   b   : 32 bytes at b   + (e*64 + lane)*32  (the B operand; 16 bytes used
 *         by the dense bf16 and int8 variants)
 *   idx : 4 bytes  at idx + (e*64 + lane)     (sparse index register)
 *   c   : 16 floats at c + (e*64 + lane)*16   (accumulator registers; 4 used
 *         by the 16x16 variants; int8 variants' int32 results converted to float)
 * n_exp >= 1.  Returns SP24_ERR_MODE for an unknown variant. */
int sp24_probe_mfma_layout(int variant, const void* a, const void* b, const uint32_t* idx,
                           float* c, int n_exp, void* stream);

/* Issue-rate loop: `blocks` workgroups of `waves` waves each issue `iters`
 * instructions of `variant` on register operands (4 independent accumulators),
 * then write one float per lane to out[(block*waves + wave)*64 + lane] so the
 * work cannot be removed.  The caller times the launch. */
int sp24_probe_mfma_rate(int variant, int iters, int blocks, int waves, float* out, void* stream);

/* Copy `bytes` (multiple of 16) from src to dst with 16-byte loads and stores:
 * the reference kernel for HBM bandwidth and for scaling traffic counters. */
int sp24_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Read `bytes` (multiple of 16) from src, writing one checksum word per
 * workgroup to out[blockIdx] (out holds >= sp24_probe_read_blocks() words):
 * the stream-read rate of HBM. */
int sp24_probe_read(const void* src, size_t bytes, uint32_t* out, void* stream);
int sp24_probe_read_blocks(void);

/* The load path of the LDS-ring GEMM kernels without their arithmetic.
 * `blocks` workgroups of 8 waves walk `steps` steps of a ring of `stages` LDS
 * buffers of (w_kb + x_kb) KB.  Per step workgroup b loads w_kb KB of W, the
 * step's next bytes of its own region w + b * w_stride (each byte once: when
 * blocks * w_stride exceeds the last-level cache, W streams from HBM), and x_kb
 * KB of X from the region x + (b % 8) * x_bytes / 8, wrapping (re-read by the
 * workgroups of each XCD, so L2-resident), with global_load_lds (16 bytes a
 * lane, W first).  Each wave waits for its loads of a step; with barrier != 0
 * the workgroup then synchronises (the GEMM kernels' ring); then the loads of
 * step + stages - 1 go out.  One checksum word per workgroup goes to out[b]
 * (out holds >= blocks words).  The caller times the launch.
 *   w: blocks * w_stride bytes, w_stride >= steps * w_kb KB, a multiple of 16;
 *   x: x_bytes, x_bytes / 8 a power of two >= x_kb KB (unused when x_kb = 0).
 * (w_kb, x_kb, stages, barrier) must be one of SP24_PROBE_RING_SHAPES (else
 * SP24_ERR_MODE): the stream kernel's mix at M = 64 (8 KB of W values and 16 KB
 * of X per step, four buffers) with and without the barrier and with six
 * buffers, and W or X alone. */
#define SP24_PROBE_RING_SHAPES(X) \
  X(8, 16, 4, true)               \
  X(8, 16, 4, false)              \
  X(8, 16, 6, true)               \
  X(8, 0, 4, true)                \
  X(24, 0, 4, true)               \
  X(0, 16, 4, true)               \
  X(0, 24, 4, true)
int sp24_probe_ring(int w_kb, int x_kb, int stages, int barrier, const void* w, size_t w_stride, const void* x,
                    size_t x_bytes, int blocks, int steps, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP24_PROBE_H */
