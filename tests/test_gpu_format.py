"""GPU parity of sp24_prune_compress and sp24_decompress against the oracle: bit-exact."""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, announce, bits, codes, need_sp, u32
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _check_prune(w_cpu, what):
    announce("prune_compress", what, tuple(w_cpu.shape))
    sp = need_sp()
    v, m = sp.prune_compress(w_cpu.to(DEV))
    torch.cuda.synchronize()
    wb = W.bf16_bits(w_cpu)
    ov, om = O.prune_compress(wb)
    gv, gm = bits(v), u32(m)
    om_stored = O.store_meta(om)
    assert np.array_equal(gm, om_stored), "%s: metadata differs in %d words" % (what, int((gm != om_stored).sum()))
    assert np.array_equal(gv, ov), "%s: values differ in %d places" % (what, int((gv != ov).sum()))
    return v, m, ov, om


def test_tiny_workload():
    _, w = W.tiny()
    _check_prune(w, "tiny")


@pytest.mark.parametrize("shape", [(1, 32), (3, 64), (5, 96), (6, 160), (17, 352), (37, 256), (5, 4096)])
def test_tie_heavy_alphabet(shape):
    rng = np.random.default_rng(sum(shape))
    vals = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0], dtype=np.float32), size=shape)
    _check_prune(torch.from_numpy(vals).to(torch.bfloat16), "alphabet")


def test_exhaustive_groups_of_small_alphabet():
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0]
    groups = np.array(list(itertools.product(alphabet, repeat=4)), dtype=np.float32)  # 2401 x 4
    pad = (-groups.shape[0]) % 8
    groups = np.concatenate([groups, np.zeros((pad, 4), np.float32)])
    w = torch.from_numpy(groups.reshape(-1, 32)).to(torch.bfloat16)
    _check_prune(w, "exhaustive alphabet")


def test_subnormal_and_extreme_magnitudes():
    rng = np.random.default_rng(7)
    pool = np.array([0.0, -0.0, 2.0 ** -133, -2.0 ** -133, 2.0 ** -126, 1e-38, 3e38, -3e38, 1.0],
                    dtype=np.float32)
    w = torch.from_numpy(rng.choice(pool, size=(64, 128))).to(torch.bfloat16)
    _check_prune(w, "subnormals")


@pytest.mark.parametrize("which", ["up", "down"])
def test_full_size_decode_weights(which):
    w = W.up_weight() if which == "up" else W.down_weight()
    _check_prune(w, which)


def test_decompress_bf16_and_fp8():
    sp = need_sp()
    _, w = W.tiny()
    w = torch.cat([w, W.randn_bf16((3, 256), seed=9)], dim=0)   # n = 259: ragged
    v, m, ov, om = _check_prune(w, "decompress input")
    announce("decompress bf16")
    d = sp.decompress(v, m, 256)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d), O.decompress(ov, om, 256))
    assert np.array_equal(bits(d), O.apply_mask(W.bf16_bits(w), O.prune_mask(W.bf16_bits(w))))
    announce("decompress fp8")
    q, s = sp.quant_fp8(v)
    d8 = sp.decompress(q, m, 256)
    torch.cuda.synchronize()
    oq, _ = O.quant_fp8(ov)
    assert np.array_equal(codes(d8), O.decompress(oq, om, 256))
    # pruning the decompressed weight again changes nothing
    v2, m2 = sp.prune_compress(d)
    torch.cuda.synchronize()
    assert np.array_equal(u32(m2), O.store_meta(om)) and np.array_equal(bits(v2), ov)


def test_decompress_random_codes_all_nibbles():
    sp = need_sp()
    rng = np.random.default_rng(3)
    n, k = 9, 192
    pairs = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    nib = np.array([a | (b << 2) for a, b in pairs], dtype=np.uint32)
    sel = rng.integers(0, 6, size=(n, k // 32, 8))
    meta = (nib[sel] << (4 * np.arange(8, dtype=np.uint32))).sum(-1).astype(np.uint32)
    vals = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    announce("decompress random codes")
    d = sp.decompress(torch.from_numpy(vals).to(DEV),
                      torch.from_numpy(O.store_meta(meta).view(np.int32)).to(DEV), k)
    torch.cuda.synchronize()
    assert np.array_equal(codes(d), O.decompress(vals, meta, k))


def test_check_meta_counts_invalid_nibbles():
    sp = need_sp()
    announce("check_meta")
    w = W.randn_bf16((96, 1024), seed=77, std=0.02)
    _, meta = sp.prune_compress(w.to(DEV))
    assert int(sp.check_meta(meta, 1024).cpu()[0]) == 0          # every written nibble is valid
    m = u32(meta).copy()
    rng = np.random.default_rng(78)
    invalid = np.array([0, 1, 2, 3, 5, 6, 7, 10, 11, 15], dtype=np.uint32)
    cells = rng.choice(m.size * 8, size=500, replace=False)         # (word, nibble) cells
    for c in cells:
        word, g = divmod(int(c), 8)
        m[word] = (m[word] & ~np.uint32(0xF << (4 * g))) | (rng.choice(invalid) << np.uint32(4 * g))
    nib = (m[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    expected = int(((nib & 3) >= (nib >> 2)).sum())                # i0 >= i1: not a kept pair
    assert expected == 500
    bad = sp.check_meta(torch.from_numpy(m.view(np.int32)).to(DEV), 1024)
    assert int(bad.cpu()[0]) == expected
    # the count is added to the given counter
    assert int(sp.check_meta(torch.from_numpy(m.view(np.int32)).to(DEV), 1024, bad).cpu()[0]) == 2 * expected
