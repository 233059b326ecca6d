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
    with their row numbers; inputs must be finite;
  * storage order in memory (``palette_store``): rows of each kind in blocks
    of 16 (the last block padded), K in chunks of 512 (the last chunk T*128
    values, T = 1..3, when K % 512 != 0); inside a (block, chunk) tile the
    16-byte pieces are ordered [piece j][lane group q][row r16], where lane
    group q holds K [32Tq, 32T(q+1)) of the chunk and piece j its j-th 16 bytes.
    One 64-lane load then reads 1 KB of consecutive memory.  The format
    needs K % 128 == 0.

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


def _tile_order(row_bytes: np.ndarray, k: int, b32: int) -> np.ndarray:
    """Storage order of compact rows [n, k/32 * b32] bytes (b32 bytes per 32 elements)."""
    n = row_bytes.shape[0]
    npad = (n + 15) // 16 * 16
    width = k // 32 * b32
    src = np.zeros((npad, width), dtype=np.uint8)
    src[:n] = row_bytes.reshape(n, width)
    out = np.zeros(npad * width, dtype=np.uint8)
    units = k // 128
    pos = 0
    for b in range(npad // 16):
        for c0 in range(0, units, 4):
            t = min(4, units - c0)
            base = c0 * 4 * b32                      # row byte offset of the chunk (4 x 32 values per unit)
            span = t * b32                           # bytes of one lane group's K range (32t values)
            for j in range(span // 16):
                for q in range(4):
                    for r16 in range(16):
                        o = base + q * span + 16 * j
                        out[pos:pos + 16] = src[16 * b + r16, o:o + 16]
                        pos += 16
    assert pos == out.size
    return out


def palette_store(enc):
    """The encoded arrays in their storage order: (sign+mantissa bytes uint8, index words
    uint32, verbatim rows uint16), each over its row count padded to a multiple of 16
    (padding zero)."""
    k = enc["k"]
    assert k % 128 == 0
    sm = _tile_order(np.asarray(enc["sm"], dtype=np.uint8), k, 32)
    ix = _tile_order(np.ascontiguousarray(enc["ix"], dtype="<u4").view(np.uint8), k, 16).view("<u4")
    verb = _tile_order(np.ascontiguousarray(enc["verb"], dtype="<u2").view(np.uint8), k, 64).view("<u2")
    return sm, ix.astype(np.uint32), verb.astype(np.uint16)


def encoded_bytes(enc) -> int:
    """Bytes of the encoded weight: palette, row lists, sign+mantissa, indices, verbatim rows."""
    n_p, n_v, k = len(enc["pal_rows"]), len(enc["verb_rows"]), enc["k"]
    return 16 + 4 * (n_p + n_v) + n_p * k + n_p * k // 2 + 2 * n_v * k   # unpadded


def gemm_ref(x_bits: np.ndarray, w_bits: np.ndarray):
    """``ref = X W^T`` and ``mag = |X| |W|^T`` in float64 of bf16 operands."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T
