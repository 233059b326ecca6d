"""On-device checks of the matrix-instruction operand layouts the GEMM kernels rely on.

Model of the sparse instructions (SMFMAC) on gfx950, measured with one-hot
probes: an instruction covers Kt values of K (fp8 and int8: 16x16x128 and
32x32x64; bf16: 16x16x64 and 32x32x32), with R rows (16 or 32) and G = 64/R
lane groups; the int8 forms share the fp8 operand layouts.
  * A (compressed): lane l holds row l % R and, for lane group q = l // R, the
    contiguous instruction-K slice [q*Kt/G, (q+1)*Kt/G); its compressed value j
    belongs to group j // 2 of the slice and the 2-bit position within the
    group is bits [2j+1:2j] of the index register (for bf16, of the 16-bit half
    selected by abid).
  * B (dense): lane l holds column l % R; its slots come in two halves of
    Kt/(2G) values, half h covering instruction K [h*Kt/2 + q*Kt/(2G), ...).
  * The accumulator layout is the dense instructions' one.
Dense instructions only need A and B to share one slot -> K map.
These tests predict the accumulator from random small-integer operands under
that model and require exact equality.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_helpers import need_sp

E4M3_SMALL = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, -1: 0xB8, -2: 0xC0, -3: 0xC4}


def _bf16_bits(v):
    return (torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))


def _c_coords(variant, lane, reg):
    """(row, col) of accumulator register `reg` of `lane`."""
    if variant in (3, 4, 5, 9, 11):  # 32x32
        return 8 * (reg // 4) + 4 * (lane // 32) + reg % 4, lane % 32
    return 4 * (lane // 16) + reg, lane % 16


def _run(variant, a_bytes, b_bytes, idx, n_exp):
    dev = torch.device("cuda:0")
    a = torch.from_numpy(a_bytes.reshape(-1)).to(dev)
    b = torch.from_numpy(b_bytes.reshape(-1)).to(dev)
    ix = torch.from_numpy(idx.reshape(-1).view(np.int32)).to(dev)
    c = torch.zeros(n_exp * 64 * 16, dtype=torch.float32, device=dev)
    need_sp().probe_mfma_layout(variant, a, b, ix, c, n_exp)
    torch.cuda.synchronize()
    return c.cpu().numpy().reshape(n_exp, 64, 16)


def _rand_idx(rng, n_exp):
    """Index words with a valid (i0 < i1) pair in every 4-bit field."""
    pairs = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    nib = np.array([i0 | (i1 << 2) for i0, i1 in pairs], dtype=np.uint32)
    sel = rng.integers(0, 6, size=(n_exp, 64, 8))
    return (nib[sel] << (4 * np.arange(8, dtype=np.uint32))).sum(-1).astype(np.uint32)


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5, 8, 9])
def test_sparse_layout(variant):
    rng = np.random.default_rng(100 + variant)
    n_exp = 8
    fp8 = variant in (0, 3, 8, 9)   # one-byte operands (E4M3 or int8)
    i8 = variant in (8, 9)
    rows = 32 if variant in (3, 4, 5, 9) else 16
    n_a = 16 if fp8 else 8         # compressed values per lane
    n_b = 32 if fp8 else 16        # B values per lane
    abid = 1 if variant in (2, 5) else 0
    av = rng.integers(-3, 4, size=(n_exp, 64, n_a))
    bv = rng.integers(-3, 4, size=(n_exp, 64, n_b))
    idx = _rand_idx(rng, n_exp)
    a_bytes = np.zeros((n_exp, 64, 32), dtype=np.uint8)
    b_bytes = np.zeros((n_exp, 64, 32), dtype=np.uint8)
    if i8:
        a_bytes[..., :16] = av.astype(np.int8).view(np.uint8)
        b_bytes[...] = bv.astype(np.int8).view(np.uint8)
    elif fp8:
        a_bytes[..., :16] = np.vectorize(E4M3_SMALL.get)(av).astype(np.uint8)
        b_bytes[...] = np.vectorize(E4M3_SMALL.get)(bv).astype(np.uint8)
    else:
        a_bytes[..., :16] = _bf16_bits(av.astype(np.float32)).view(np.uint8).reshape(n_exp, 64, 16)
        b_bytes[...] = _bf16_bits(bv.astype(np.float32)).view(np.uint8).reshape(n_exp, 64, 32)
    got = _run(variant, a_bytes, b_bytes, idx, n_exp)
    groups = 64 // rows
    kt = (n_a * 2) * groups          # instruction K
    half = kt // (2 * groups)        # B values per half-slot run
    for e in range(n_exp):
        want = np.zeros((rows, rows))
        # dense B[k, col] from the lane layout
        bdense = np.zeros((kt, rows))
        for l in range(64):
            q, col = l // rows, l % rows
            for s_ in range(n_b):
                h, o = s_ // half, s_ % half
                bdense[h * kt // 2 + q * half + o, col] = bv[e, l, s_]
        for l in range(64):
            q, i = l // rows, l % rows
            bits = int(idx[e, l]) >> (16 * abid) if not fp8 else int(idx[e, l])
            for j in range(n_a):
                pos = (bits >> (2 * j)) & 3
                k = q * (kt // groups) + 4 * (j // 2) + pos
                want[i, :] += av[e, l, j] * bdense[k, :]
        nreg = 16 if rows == 32 else 4
        for l in range(64):
            for r in range(nreg):
                i, col = _c_coords(variant, l, r)
                assert got[e, l, r] == want[i, col], (variant, e, l, r)


@pytest.mark.parametrize("variant", [6, 7, 10, 11])
def test_dense_layout_consistency(variant):
    rng = np.random.default_rng(200 + variant)
    n_exp = 4
    fp8 = variant == 6
    i8 = variant in (10, 11)
    rows = 32 if variant == 11 else 16
    n = 32 if fp8 else 16 if i8 else 8
    av = rng.integers(-3, 4, size=(n_exp, 64, n))
    bv = rng.integers(-3, 4, size=(n_exp, 64, n))
    a_bytes = np.zeros((n_exp, 64, 32), dtype=np.uint8)
    b_bytes = np.zeros((n_exp, 64, 32), dtype=np.uint8)
    if i8:
        a_bytes[..., :16] = av.astype(np.int8).view(np.uint8)
        b_bytes[..., :16] = bv.astype(np.int8).view(np.uint8)
    elif fp8:
        a_bytes[...] = np.vectorize(E4M3_SMALL.get)(av).astype(np.uint8)
        b_bytes[...] = np.vectorize(E4M3_SMALL.get)(bv).astype(np.uint8)
    else:
        a_bytes[..., :16] = _bf16_bits(av.astype(np.float32)).view(np.uint8).reshape(n_exp, 64, 16)
        b_bytes[..., :16] = _bf16_bits(bv.astype(np.float32)).view(np.uint8).reshape(n_exp, 64, 16)
    idx = np.zeros((n_exp, 64), dtype=np.uint32)
    got = _run(variant, a_bytes, b_bytes, idx, n_exp)
    for e in range(n_exp):
        want = np.zeros((rows, rows))
        for q in range(64 // rows):
            want += av[e, rows * q:rows * q + rows] @ bv[e, rows * q:rows * q + rows].T
        for l in range(64):
            for r in range(16 if rows == 32 else 4):
                i, col = _c_coords(variant, l, r)
                assert got[e, l, r] == want[i, col], (variant, e, l, r)
