"""CPU oracle for 2:4 structured-sparse GEMM (prune, compress, FP8 quantise, GEMM).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library and imports nothing from it.  It is deliberately plain and slow:
NumPy, exact integer work on bit patterns, IEEE float32 where the method fixes
float32, and float64 for the reference product.

Sources ("the cookbook" = the page "Deploying 2:4 Sparsity with FP8 on Hopper:
A Production Cookbook"):

* 2:4 pruning: the cookbook, pipeline step 4 "Apply 2:4 structured pruning
  safely" (keep the two largest-magnitude values of every 4) and step 2
  "Choose 2:4-eligible layers and orientation" (groups are 4 contiguous values
  along the inner K dimension); Practical Example 1 "2:4 mask application" (a
  top-2-of-|w| mask over groups of 4 along the chosen axis; the axis length must
  be divisible by 4).
* Compressed form: kept values plus 2-bit positions; the SlideSparse page
  ("SlideSparse: Fast and Flexible (2N-2):2N Structured Sparsity") describes the
  weights being converted once, offline, into the hardware's compressed format.
* FP8 scaling: the cookbook, pipeline step 3 "Calibrate for FP8 and sparsity"
  (per-tensor dynamic scaling to avoid overflow), step 6 "Precision pipeline and
  post-pruning recalibration" (scales recomputed after pruning) and
  "Troubleshooting quick hits" (clip the maximum to avoid overflow and NaN).
* Readings where the pages are silent (each is applied below and nowhere else):
  ties in |w| go to the lower index; magnitudes are compared exactly on the
  bfloat16 bit patterns (+0 and -0 equal); dropped positions decompress to +0;
  kept values are stored in ascending index order; position nibble
  ``i0 | i1 << 2`` for group g sits at bits ``4*(g % 8)`` of metadata word
  ``g // 8``; FP8 is OCP E4M3FN (bias 7, max 448, no infinities, NaN = S.1111.111);
  the scale is ``s = fp32(amax / 448)`` (``s = 1`` when amax is 0) and a value is
  quantised as ``e4m3_rne(clamp(fp32(v / s), -448, 448))``.

* INT8 W8A8: the cookbook's table "Precision and sparsity recipes" and its
  step 6 "INT8 alternative"; symmetric per-tensor scale ``fp32(amax / 127)``
  and codes ``clamp(round_half_even(fp32(v / s)), -127, 127)`` are a reading.

Representation: bfloat16 tensors are passed as ``numpy.uint16`` bit patterns,
FP8-E4M3 tensors as ``numpy.uint8`` codes, metadata as ``numpy.uint32`` words.

Parity pins live in ``tests/test_oracle_*.py``; every function here is pinned.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GROUP = 4          # values per 2:4 group along K
KEEP = 2           # kept values per group
GROUPS_PER_WORD = 8  # 4-bit position nibbles per 32-bit metadata word

# ----------------------------------------------------------------------------
# bfloat16 bit patterns
# ----------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (the high 16 bits)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------------------
# 2:4 magnitude pruning (the cookbook, pipeline step 4 and Practical Example 1)
# ----------------------------------------------------------------------------


def prune_mask(w_bits: np.ndarray) -> np.ndarray:
    """Boolean keep-mask of 2:4 magnitude pruning along the last axis (K).

    In every group of 4 contiguous values along K, value i is kept iff fewer
    than two values of the group rank above it, where j ranks above i when
    |w_j| > |w_i|, or |w_j| == |w_i| and j < i (ties go to the lower index).
    |w| is compared exactly as the unsigned integer ``bits & 0x7FFF``, which
    orders finite bfloat16 magnitudes exactly and makes +0 equal to -0.
    Inputs must be finite.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n, k = w_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 4")
    a = (w_bits & np.uint16(0x7FFF)).astype(np.int32).reshape(n, k // GROUP, GROUP)
    above = np.zeros(a.shape, dtype=np.int32)
    for i in range(GROUP):
        for j in range(GROUP):
            if j == i:
                continue
            beats = a[..., j] > a[..., i]
            if j < i:
                beats = beats | (a[..., j] == a[..., i])
            above[..., i] += beats
    return (above < KEEP).reshape(n, k)


def apply_mask(w_bits: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Pruned dense weight: kept values as they are, dropped positions +0."""
    return np.where(mask, np.asarray(w_bits, dtype=np.uint16), np.uint16(0)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Compressed 2:4 form: kept values + 2-bit positions
# ----------------------------------------------------------------------------


def compress(w: np.ndarray, mask: np.ndarray):
    """Pack the kept values of each group and their positions.

    ``w`` is ``[N, K]`` (any element type: bfloat16 bits or FP8 codes), ``mask``
    the keep-mask with exactly two True per group of 4.  Returns
    ``values [N, K/2]`` (same element type as ``w``; the two kept values of group
    g at columns 2g and 2g+1, in ascending position order) and
    ``meta [N, K/32]`` uint32 (group g's nibble ``i0 | i1 << 2`` with i0 < i1 at
    bits ``4*(g % 8)`` of word ``g // 8``).
    """
    w = np.asarray(w)
    mask = np.asarray(mask, dtype=bool)
    n, k = w.shape
    if k % (GROUP * GROUPS_PER_WORD):
        raise ValueError("K must be a multiple of 32")
    g = mask.reshape(n, k // GROUP, GROUP)
    if not np.all(g.sum(axis=-1) == KEEP):
        raise ValueError("mask must keep exactly 2 of every 4")
    i0 = np.argmax(g, axis=-1)                       # first kept position
    i1 = (GROUP - 1) - np.argmax(g[..., ::-1], axis=-1)  # last kept position
    wg = w.reshape(n, k // GROUP, GROUP)
    v0 = np.take_along_axis(wg, i0[..., None], axis=-1)[..., 0]
    v1 = np.take_along_axis(wg, i1[..., None], axis=-1)[..., 0]
    values = np.stack([v0, v1], axis=-1).reshape(n, k // 2).astype(w.dtype)
    nib = (i0 | (i1 << 2)).astype(np.uint32).reshape(n, k // 32, GROUPS_PER_WORD)
    shifts = (4 * np.arange(GROUPS_PER_WORD, dtype=np.uint32))
    meta = np.bitwise_or.reduce(nib << shifts, axis=-1).astype(np.uint32)
    return values, meta


def meta_positions(meta: np.ndarray, k: int):
    """Decode metadata words into the two kept positions (i0, i1) of every group."""
    meta = np.asarray(meta, dtype=np.uint32)
    n = meta.shape[0]
    shifts = (4 * np.arange(GROUPS_PER_WORD, dtype=np.uint32))
    nib = ((meta[..., None] >> shifts) & np.uint32(0xF)).reshape(n, k // GROUP)
    return (nib & 3).astype(np.int64), (nib >> 2).astype(np.int64)


def mask_from_meta(meta: np.ndarray, k: int) -> np.ndarray:
    i0, i1 = meta_positions(meta, k)
    n = i0.shape[0]
    m = np.zeros((n, k // GROUP, GROUP), dtype=bool)
    np.put_along_axis(m, i0[..., None], True, axis=-1)
    np.put_along_axis(m, i1[..., None], True, axis=-1)
    return m.reshape(n, k)


def decompress(values: np.ndarray, meta: np.ndarray, k: int) -> np.ndarray:
    """Inverse of :func:`compress`: dense ``[N, K]`` with zero bits at dropped positions."""
    values = np.asarray(values)
    n = values.shape[0]
    i0, i1 = meta_positions(meta, k)
    vg = values.reshape(n, k // GROUP, KEEP)
    out = np.zeros((n, k // GROUP, GROUP), dtype=values.dtype)
    np.put_along_axis(out, i0[..., None], vg[..., 0:1], axis=-1)
    np.put_along_axis(out, i1[..., None], vg[..., 1:2], axis=-1)
    return out.reshape(n, k)


def prune_compress(w_bits: np.ndarray):
    """Prune then compress a bfloat16 weight: returns (values, meta)."""
    return compress(np.asarray(w_bits, dtype=np.uint16), prune_mask(w_bits))


# Storage order of the metadata words.  The words of a row are cut into blocks
# of 4 (128 values of K); block b holds, row after row, every row's words of
# that block, and a last block of fewer than 4 words (K not a multiple of 128)
# does the same with its narrower rows.  The pages leave the layout of the
# compressed form to the implementation (the SlideSparse page has weights
# converted once, offline, into the hardware's format).
META_BLOCK_WORDS = 4


def meta_word_index(n: int, k: int, rows=None):
    """Storage index of word w of row r, as an ``[N, K/32]`` array (or for ``rows`` only)."""
    words = k // 32
    r = (np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    w = np.arange(words, dtype=np.int64)[None, :]
    b = w // META_BLOCK_WORDS
    width = np.minimum(META_BLOCK_WORDS, words - META_BLOCK_WORDS * b)
    return META_BLOCK_WORDS * n * b + r * width + (w - META_BLOCK_WORDS * b)


def store_meta(meta: np.ndarray) -> np.ndarray:
    """Metadata ``[N, K/32]`` in storage order (a flat array of N*K/32 words)."""
    meta = np.asarray(meta, dtype=np.uint32)
    n, words = meta.shape
    out = np.zeros(n * words, dtype=np.uint32)
    out[meta_word_index(n, 32 * words)] = meta
    return out


def load_meta(stored: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """Inverse of :func:`store_meta`: the ``[N, K/32]`` words of a stored array
    (or the words of ``rows`` only)."""
    stored = np.asarray(stored, dtype=np.uint32).reshape(-1)
    if stored.size != n * (k // 32):
        raise ValueError("stored metadata has %d words, expected %d" % (stored.size, n * (k // 32)))
    return stored[meta_word_index(n, k, rows)]


# ----------------------------------------------------------------------------
# FP8 E4M3 (OCP "E4M3FN": bias 7, no infinities, max finite 448)
# ----------------------------------------------------------------------------


def e4m3_value_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF).

    Code = s.eeee.mmm; e == 0 is subnormal, m/8 * 2^-6; otherwise
    (1 + m/8) * 2^(e-7); e == 15 with m == 7 is NaN.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_value_table()
_E4M3_POS = _E4M3[:0x7F]  # codes 0x00..0x7E: the non-negative finite values, ascending


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 codes: clamp to [-448, 448], then nearest, ties to even.

    The nearest code is found by searching the table of the 127 non-negative
    finite values; when |t| lies strictly between two neighbours lo < hi it
    rounds down iff 2|t| < lo + hi, up iff 2|t| > lo + hi, and to the code with
    an even (zero) last mantissa bit on equality.  Both sides of that comparison
    are exact in float64.  The sign bit is copied from t (so -0 -> 0x80).
    Inputs must not be NaN.
    """
    t = np.asarray(t, dtype=np.float32)
    if np.isnan(t).any():
        raise ValueError("NaN input")
    a = np.minimum(np.abs(t).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # _E4M3_POS[hi] >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    exact = _E4M3_POS[hi] == a
    lo = np.maximum(hi - 1, 0)
    twice = 2.0 * a
    mid = _E4M3_POS[lo] + _E4M3_POS[hi]
    pick_hi = (twice > mid) | ((twice == mid) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return code | (np.signbit(t).astype(np.uint8) << np.uint8(7))


def fp8_scale(v_bits: np.ndarray) -> np.float32:
    """Per-tensor dynamic scale ``fp32(amax / 448)``, or 1 when the tensor is all zero.

    amax is the exact maximum of |v| over the whole tensor (the cookbook, step 3:
    one scale per tensor, from the data, chosen so nothing overflows).
    """
    amax = np.float32(np.max(np.abs(bf16_to_f32(v_bits)))) if np.size(v_bits) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(E4M3_MAX)


def quant_fp8(v_bits: np.ndarray, scale=None):
    """Quantise bfloat16 values to E4M3 codes with one per-tensor scale.

    ``scale=None`` is the dynamic mode (scale from :func:`fp8_scale`); otherwise
    the given float32 scale is used as is (static mode, where the clamp at +-448
    is what keeps out-of-range values finite).  Each value is divided by the
    scale in IEEE float32 and rounded with :func:`e4m3_encode`.
    Returns (codes, scale).
    """
    s = fp8_scale(v_bits) if scale is None else np.float32(scale)
    t = bf16_to_f32(v_bits) / s
    assert t.dtype == np.float32
    return e4m3_encode(t), s


def dequant_fp8(codes: np.ndarray, scale) -> np.ndarray:
    """float64 values ``scale * decode(code)`` represented by E4M3 codes."""
    return np.float64(np.float32(scale)) * e4m3_decode(codes)


# ----------------------------------------------------------------------------
# INT8 W8A8 (symmetric, per tensor): the cookbook's table "Precision and
# sparsity recipes" lists INT8 W8A8 beside 2:4 + FP8, its pipeline step 6 "INT8
# alternative" re-quantises after pruning, and the SlideSparse page reports INT8
# results.  No page fixes the INT8 rounding; the reading taken is the FP8 recipe
# with the format's range: s = fp32(amax / 127) (1 for an all-zero tensor),
# q = clamp(round_half_even(fp32(v / s)), -127, 127) (never -128).
# ----------------------------------------------------------------------------

INT8_MAX = 127.0


def int8_scale(v_bits: np.ndarray) -> np.float32:
    """Per-tensor INT8 scale ``fp32(amax / 127)``, or 1 when the tensor is all zero."""
    amax = np.float32(np.max(np.abs(bf16_to_f32(v_bits)))) if np.size(v_bits) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(INT8_MAX)


def quant_int8(v_bits: np.ndarray, scale=None):
    """INT8 codes of bfloat16 values: ``clamp(rne(fp32(v / s)), -127, 127)``, dynamic
    (``scale=None``) or static scale.  Returns (codes int8, scale)."""
    s = int8_scale(v_bits) if scale is None else np.float32(scale)
    t = bf16_to_f32(v_bits) / s
    assert t.dtype == np.float32
    r = np.rint(t)                               # IEEE round to nearest, ties to even
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8), s


def dequant_int8(codes: np.ndarray, scale) -> np.ndarray:
    """float64 values ``scale * code`` of INT8 codes."""
    return np.float64(np.float32(scale)) * np.asarray(codes, dtype=np.int8).astype(np.float64)


def sparse_operands_int8(xq, x_scale, wq_values, meta, w_scale, k):
    """Dense float64 operands of the INT8 path: both dequantised, W decompressed."""
    return dequant_int8(xq, x_scale), dequant_int8(decompress(wq_values, meta, k), w_scale)


def quant_int8_rows(x_bits: np.ndarray):
    """Per-token INT8: row m quantised on its own, ``quant_int8(x[m])``.
    Returns (codes int8 [M, K], scales float32 [M])."""
    x = np.asarray(x_bits, dtype=np.uint16)
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[0], dtype=np.float32)
    for m in range(x.shape[0]):
        codes[m], scales[m] = quant_int8(x[m])
    return codes, scales


def sparse_operands_int8_rows(xq, x_scales, wq_values, meta, w_scale, k):
    """Dense float64 operands of the INT8 path with one scale per X row."""
    xs = np.asarray(x_scales, dtype=np.float32).astype(np.float64)[:, None]
    return xs * np.asarray(xq, dtype=np.int8).astype(np.float64), dequant_int8(decompress(wq_values, meta, k),
                                                                                 w_scale)


def quant_fp8_rows(x_bits: np.ndarray):
    """Quantise each row (token) of X ``[M, K]`` with its own dynamic scale.

    The per-token quantisation the SlideSparse page ("SlideSparse: Fast and
    Flexible (2N-2):2N Structured Sparsity", activation lifting) fuses its
    activation step into, and the finer scales the page "La Densite Dynamique et
    les Noyaux Non Structures ..." recommends for outlier-heavy layers: row m is
    quantised exactly as :func:`quant_fp8` would quantise that row alone.
    Returns (codes ``[M, K]``, scales ``[M]`` float32).
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[0], dtype=np.float32)
    for m in range(x.shape[0]):
        codes[m], scales[m] = quant_fp8(x[m])
    return codes, scales


def dequant_fp8_rows(codes: np.ndarray, scales) -> np.ndarray:
    """float64 values ``scales[m] * decode(code)`` of row-scaled E4M3 codes."""
    return np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None] * e4m3_decode(codes)


# ----------------------------------------------------------------------------
# Finer FP8 scales: one scale per group of consecutive values of a row.  The
# research-roadmap page ("La Densite Dynamique et les Noyaux Non Structures",
# quantisation under extreme sparsity) recommends per-channel or per-group
# scales for outlier-heavy layers.  No page fixes the details; the readings:
#   * a group is `group` consecutive values of one row; each group is quantised
#     exactly as quant_fp8 would quantise it alone (s = fp32(amax / 448), 1 for
#     an all-zero group; codes by IEEE float32 division and round to nearest
#     even);
#   * X [M, K] takes groups along K; the weight takes them along its compressed
#     rows [N, K/2], group/2 kept values for a group of K values (the kept values
#     of K positions [group*g, group*(g+1)) are compressed columns
#     [group/2*g, group/2*(g+1)));
#   * one group per row is per-token X and per-output-channel W;
#   * the product is sum_k (s_x[m, k // group] dec(qx)) (s_w[n, k // group] dec(qw)),
#     which the float64 reference below takes as written.
# ----------------------------------------------------------------------------


def fp8_group_scales(v_bits: np.ndarray, group: int) -> np.ndarray:
    """Dynamic scales of each group of ``group`` consecutive values of every row of
    ``v [R, C]``: ``fp32(amax / 448)`` per group, 1 for an all-zero group.
    Returns float32 ``[R, C // group]``."""
    v = np.asarray(v_bits, dtype=np.uint16)
    rows, cols = v.shape
    if group < 1 or cols % group:
        raise ValueError("the row length must be a multiple of the group")
    amax = np.max(np.abs(bf16_to_f32(v)).reshape(rows, cols // group, group), axis=2).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)


def quant_fp8_groups(v_bits: np.ndarray, group: int):
    """Quantise ``v [R, C]`` (bfloat16 bits) with one dynamic scale per group of
    ``group`` consecutive values of a row: every group exactly as :func:`quant_fp8`
    would quantise it alone.  Returns (codes uint8 ``[R, C]``, scales float32
    ``[R, C // group]``)."""
    v = np.asarray(v_bits, dtype=np.uint16)
    scales = fp8_group_scales(v, group)
    t = bf16_to_f32(v) / np.repeat(scales, group, axis=1)
    assert t.dtype == np.float32
    return e4m3_encode(t), scales


def dequant_fp8_groups(codes: np.ndarray, scales, group: int) -> np.ndarray:
    """float64 values ``scales[r, c // group] * decode(code[r, c])``."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return np.repeat(s, group, axis=1) * e4m3_decode(codes)


def sparse_operands_fp8_groups(xq, x_scales, wq_values, meta, w_scales, k: int, group: int):
    """Dense float64 operands of the FP8 path with group scales: X ``[M, K]`` codes with
    ``x_scales [M, K // group]``; W compressed codes ``[N, K/2]`` with ``w_scales
    [N, K // group]`` (each over group/2 kept values), decompressed to ``[N, K]``
    (dropped positions are code 0, i.e. +0) and scaled by the group of their K position."""
    x_hat = dequant_fp8_groups(xq, x_scales, group)
    w_hat = dequant_fp8_groups(decompress(wq_values, meta, k), w_scales, group)
    return x_hat, w_hat


# ----------------------------------------------------------------------------
# Reference product Y = X . W^T (float64) and its magnitude sum
# ----------------------------------------------------------------------------


def gemm_ref(x_hat: np.ndarray, w_hat: np.ndarray):
    """``ref = X W^T`` and ``mag = |X| |W|^T`` in float64.

    ``x_hat`` is ``[M, K]``, ``w_hat`` ``[N, K]`` (dense, pruned, dequantised).
    ``mag[m, n] = sum_k |x[m,k] w[n,k]|`` scales the accumulation-order part of
    the tolerance.
    """
    x_hat = np.asarray(x_hat, dtype=np.float64)
    w_hat = np.asarray(w_hat, dtype=np.float64)
    return x_hat @ w_hat.T, np.abs(x_hat) @ np.abs(w_hat).T


def sparse_operands_bf16(x_bits, values, meta, k):
    """Dense float64 operands of the BF16 path: X as given, W decompressed."""
    return bf16_to_f64(x_bits), bf16_to_f64(decompress(values, meta, k))


def sparse_operands_fp8(xq, x_scale, wq_values, meta, w_scale, k):
    """Dense float64 operands of the FP8 path: both dequantised, W decompressed."""
    return dequant_fp8(xq, x_scale), dequant_fp8(decompress(wq_values, meta, k), w_scale)


def sparse_operands_fp8_rows(xq, x_scales, wq_values, meta, w_scale, k):
    """Dense float64 operands of the FP8 path with one scale per X row."""
    return dequant_fp8_rows(xq, x_scales), dequant_fp8(decompress(wq_values, meta, k), w_scale)


def within_tolerance(y, ref, mag, rel=8e-3, absmag=1e-4):
    """Elementwise test ``|y - ref| <= rel*|ref| + absmag*mag`` (y: the BF16 output as float)."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - ref) <= rel * np.abs(ref) + absmag * mag


# ----------------------------------------------------------------------------
# SlideSparse: (2N-2):2N weights on 2:4 hardware ("SlideSparse: Fast and
# Flexible (2N-2):2N Structured Sparsity", technical summary, section 2)
# ----------------------------------------------------------------------------


def slide_prune_mask(w_bits: np.ndarray, n_pat: int) -> np.ndarray:
    """Keep the 2N-2 largest |w| of every block of 2N along K (ties to the lower
    index, exact bf16 magnitudes, as for 2:4): the (2N-2):2N pattern."""
    w = np.asarray(w_bits, dtype=np.uint16)
    rows, k = w.shape
    blk = 2 * n_pat
    if k % blk:
        raise ValueError("K must be a multiple of 2N")
    a = (w & np.uint16(0x7FFF)).astype(np.int64).reshape(rows, k // blk, blk)
    # rank of each value: how many beat it (larger, or equal at a lower index)
    rank = np.zeros(a.shape, dtype=np.int64)
    for i in range(blk):
        for j in range(blk):
            if i == j:
                continue
            beats = (a[..., j] > a[..., i]) | ((a[..., j] == a[..., i]) & (j < i))
            rank[..., i] += beats
    return (rank < blk - 2).reshape(rows, k)


def slide_windows(nonzero: np.ndarray, n_pat: int):
    """Assign the nonzero positions of one block of 2N to the N-1 windows of 4
    at stride 2 (window j covers block positions 2j .. 2j+3), at most 2 per
    window.  Window j first takes what no later window can (positions 2j,
    2j+1), then fills up from positions 2j+2, 2j+3 in ascending order; what it
    cannot hold spills into the next window.  Returns the window of every
    position (-1 for zeros); raises if the block does not fit."""
    nz = [bool(v) for v in nonzero]
    if len(nz) != 2 * n_pat:
        raise ValueError("a block holds 2N values")
    owner = [-1] * (2 * n_pat)
    for j in range(n_pat - 1):
        must = [p for p in (2 * j, 2 * j + 1) if nz[p] and owner[p] < 0]
        last = j == n_pat - 2
        may = [p for p in (2 * j + 2, 2 * j + 3) if nz[p] and owner[p] < 0]
        if last:
            must += may
            may = []
        if len(must) > 2:
            raise ValueError("block has more than 2N-2 nonzeros that fit: %s" % nonzero)
        take = must + may[: 2 - len(must)]
        for p in take:
            owner[p] = j
    return owner


def slide_pack(w: np.ndarray, n_pat: int) -> np.ndarray:
    """The expanded weight W' [rows, K * (2N-2)/N] of a (2N-2):2N weight: block b
    of 2N values becomes N-1 groups of 4, group j holding the values its window
    owns at window positions 0..3 and zero elsewhere (any element type; zero
    bits are the zero value)."""
    w = np.asarray(w)
    rows, k = w.shape
    blk, grp = 2 * n_pat, 4 * (n_pat - 1)
    out = np.zeros((rows, k // blk * grp), dtype=w.dtype)
    zero = np.zeros((), dtype=w.dtype)
    for r in range(rows):
        for b in range(k // blk):
            block = w[r, b * blk:(b + 1) * blk]
            owner = slide_windows(block != zero, n_pat)
            for p, j in enumerate(owner):
                if j >= 0:
                    out[r, b * grp + 4 * j + (p - 2 * j)] = block[p]
    return out


def slide_lift(x: np.ndarray, n_pat: int) -> np.ndarray:
    """Activation lifting: X' [M, K * (2N-2)/N] with X'[m, b*4(N-1) + 4j + p] =
    X[m, b*2N + 2j + p], so that X' W'^T = X W^T (any element type)."""
    x = np.asarray(x)
    rows, k = x.shape
    blk, grp = 2 * n_pat, 4 * (n_pat - 1)
    idx = np.array([b * blk + 2 * j + p for b in range(k // blk) for j in range(n_pat - 1) for p in range(4)])
    assert idx.size == k // blk * grp
    return x[:, idx]
