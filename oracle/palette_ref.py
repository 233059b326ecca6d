"""CPU oracle for the lossless BF16 exponent-palette weight format and its GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library and imports nothing from it.  NumPy on bfloat16 bit patterns
(``numpy.uint16``); no floating point except the float64 reference product.

Source: the page "Unweight: Compresion Lossless de Pesos de LLM para Inferencia
en GPU H100", sections on the architecture (the 8 exponent bits of a BF16
weight are the redundant part, sign and 7-bit mantissa stay as they are; the 16
most common exponents cover almost every weight; weight rows with an exponent
outside that 16-entry palette are stored verbatim, so the hot path never
branches per element) and on the execution pipelines (the "direct palette"
pipeline transcodes to 4-bit palette indices at load time and the matmul kernel
rebuilds BF16 on chip; the "full decode" pipeline rebuilds BF16 in memory and
runs a standard GEMM).

Readings where the page is silent (each applied below and nowhere else):
  * one palette per weight tensor; its entries are the exponents ranked by
    count, most frequent first, ties to the smaller exponent; only exponents
    that occur are entries; unused entries hold 0xFF (the exponent of Inf/NaN,
    which a finite weight never has);
  * a row is verbatim when any of its exponents is not in the palette;
  * paletted element -> one byte ``sign << 7 | mantissa`` and a 4-bit index
    (the position of its exponent in the palette);
  * index storage: one 32-bit word per 8 consecutive elements of a row; element
    8g + t (t < 4) at bits [8t, 8t + 4), element 8g + 4 + t at bits
    [8t + 4, 8t + 8);
  * paletted and verbatim rows are stored compactly in ascending row order
    with their row numbers; inputs must be finite.

Every function is pinned in ``tests/test_oracle_palette.py``.
"""
from __future__ import annotations

import numpy as np

PALETTE_SIZE = 16
UNUSED = 0xFF


def exponent(bits: np.ndarray) -> np.ndarray:
    """The 8 exponent bits of bfloat16 bit patterns."""
    return ((np.asarray(bits, dtype=np.uint16) >> np.uint16(7)) & np.uint16(0xFF)).astype(np.uint8)


def palette_select(w_bits: np.ndarray) -> np.ndarray:
    """The 16-entry palette: exponents by count (descending), ties to the smaller exponent."""
    counts = np.bincount(exponent(w_bits).ravel().astype(np.int64), minlength=256)
    present = [e for e in range(256) if counts[e] > 0]
    ranked = sorted(present, key=lambda e: (-int(counts[e]), e))
    pal = np.full(PALETTE_SIZE, UNUSED, dtype=np.uint8)
    for i, e in enumerate(ranked[:PALETTE_SIZE]):
        pal[i] = e
    return pal


def pack_indices(idx: np.ndarray) -> np.ndarray:
    """4-bit indices [rows, k] (k % 8 == 0) -> uint32 words [rows, k/8] in the storage order."""
    idx = np.asarray(idx, dtype=np.uint32)
    rows, k = idx.shape
    g = idx.reshape(rows, k // 8, 8)
    words = np.zeros((rows, k // 8), dtype=np.uint32)
    for t in range(4):
        words |= g[:, :, t] << np.uint32(8 * t)
        words |= g[:, :, 4 + t] << np.uint32(8 * t + 4)
    return words


def unpack_indices(words: np.ndarray, k: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    rows = words.shape[0]
    idx = np.zeros((rows, k // 8, 8), dtype=np.uint8)
    for t in range(4):
        idx[:, :, t] = (words >> np.uint32(8 * t)) & np.uint32(15)
        idx[:, :, 4 + t] = (words >> np.uint32(8 * t + 4)) & np.uint32(15)
    return idx.reshape(rows, k)


def palette_encode(w_bits: np.ndarray):
    """Encode W [n, k] (bf16 bits, k % 8 == 0).

    Returns a dict: palette uint8[16]; pal_rows int32[n_p]; sm uint8[n_p, k]
    (sign << 7 | mantissa); ix uint32[n_p, k/8]; verb_rows int32[n_v];
    verb uint16[n_v, k] (the rows' bits unchanged)."""
    w = np.asarray(w_bits, dtype=np.uint16)
    n, k = w.shape
    assert k % 8 == 0
    pal = palette_select(w)
    where = np.full(256, -1, dtype=np.int64)         # exponent -> palette index
    for i in range(PALETTE_SIZE):
        if pal[i] != UNUSED:
            where[pal[i]] = i
    e = exponent(w).astype(np.int64)
    idx = where[e]
    verbatim = (idx < 0).any(axis=1)
    pal_rows = np.flatnonzero(~verbatim).astype(np.int32)
    verb_rows = np.flatnonzero(verbatim).astype(np.int32)
    wp = w[pal_rows]
    sm = (((wp >> np.uint16(8)) & np.uint16(0x80)) | (wp & np.uint16(0x7F))).astype(np.uint8)
    ix = pack_indices(idx[pal_rows].astype(np.uint8)) if len(pal_rows) else np.zeros((0, k // 8), np.uint32)
    return {"palette": pal, "pal_rows": pal_rows, "sm": sm, "ix": ix,
            "verb_rows": verb_rows, "verb": w[verb_rows].copy(), "n": n, "k": k}


def palette_decode(enc) -> np.ndarray:
    """Rebuild W [n, k] (bf16 bits) from palette_encode's output."""
    n, k = enc["n"], enc["k"]
    w = np.zeros((n, k), dtype=np.uint16)
    if len(enc["pal_rows"]):
        sm = enc["sm"].astype(np.uint16)
        e = enc["palette"][unpack_indices(enc["ix"], k)].astype(np.uint16)
        w[enc["pal_rows"]] = ((sm & np.uint16(0x80)) << np.uint16(8)) | (e << np.uint16(7)) | (sm & np.uint16(0x7F))
    w[enc["verb_rows"]] = enc["verb"]
    return w


def encoded_bytes(enc) -> int:
    """Bytes of the encoded weight: palette, row lists, sign+mantissa, indices, verbatim rows."""
    n_p, n_v, k = len(enc["pal_rows"]), len(enc["verb_rows"]), enc["k"]
    return 16 + 4 * (n_p + n_v) + n_p * k + n_p * k // 2 + 2 * n_v * k


def gemm_ref(x_bits: np.ndarray, w_bits: np.ndarray):
    """``ref = X W^T`` and ``mag = |X| |W|^T`` in float64 of bf16 operands."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T
