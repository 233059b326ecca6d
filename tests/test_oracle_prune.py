"""Pins for the oracle's 2:4 pruning, compression and decompression.

Pruning follows the cookbook page ("Deploying 2:4 Sparsity with FP8 on Hopper"),
pipeline step 4 and Practical Example 1: keep the two largest |w| of every 4
contiguous values along K.  Ties go to the lower index (the reading used by
this library; the page's top-2 selection leaves tie order open).
"""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O


def _bf16_bits_of(vals):
    t = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    return W.bf16_bits(t)


def _brute_keep(a):
    """Best pair by (larger magnitude, smaller magnitude); on equal keys the
    lexicographically smallest index pair.  Independent of the ranking count."""
    best = None
    for i, j in itertools.combinations(range(4), 2):
        key = (max(a[i], a[j]), min(a[i], a[j]))
        if best is None or key > best[0]:
            best = (key, (i, j))
    return best[1]


def _sorted_keep(a):
    """Definition by sorting: order by magnitude descending, index ascending."""
    order = sorted(range(4), key=lambda i: (-a[i], i))
    return tuple(sorted(order[:2]))


def test_exhaustive_small_alphabet_matches_brute_force():
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0]
    groups = np.array(list(itertools.product(alphabet, repeat=4)), dtype=np.float32)
    bits = _bf16_bits_of(groups)  # [8^4, 4]
    mask = O.prune_mask(bits)
    mags = (bits & 0x7FFF).astype(np.int64)
    for g in range(bits.shape[0]):
        a = mags[g].tolist()
        want = _brute_keep(a)
        assert want == _sorted_keep(a)
        got = tuple(np.nonzero(mask[g])[0].tolist())
        assert got == want, (groups[g], got, want)


def test_subnormal_and_signed_zero_mixes():
    tiny = float(torch.tensor(2.0 ** -133).to(torch.bfloat16))  # bf16 subnormal
    assert tiny != 0.0
    alphabet = [0.0, -0.0, tiny, -tiny, 2 * tiny, 1e-38]
    groups = np.array(list(itertools.product(alphabet, repeat=4)), dtype=np.float32)
    bits = _bf16_bits_of(groups)
    mask = O.prune_mask(bits)
    mags = (bits & 0x7FFF).astype(np.int64)
    for g in range(bits.shape[0]):
        assert tuple(np.nonzero(mask[g])[0].tolist()) == _sorted_keep(mags[g].tolist())


def test_invariants_random(rng):
    x = torch.from_numpy(rng.standard_normal((37, 256)).astype(np.float32)) * 0.02
    bits = W.bf16_bits(x.to(torch.bfloat16))
    mask = O.prune_mask(bits)
    g = mask.reshape(37, 64, 4)
    assert np.all(g.sum(-1) == 2)
    mag = np.abs(O.bf16_to_f64(bits)).reshape(37, 64, 4)
    kept_min = np.where(g, mag, np.inf).min(-1)
    drop_max = np.where(~g, mag, -np.inf).max(-1)
    assert np.all(kept_min >= drop_max)
    pruned = O.apply_mask(bits, mask)
    # the group maximum is always kept, so amax is unchanged by pruning
    assert np.abs(O.bf16_to_f64(pruned)).max() == np.abs(O.bf16_to_f64(bits)).max()
    # idempotent
    assert np.array_equal(O.prune_mask(pruned), mask)
    # dropped positions are +0 (no -0 bit patterns)
    assert np.all(pruned[~mask] == 0)


def test_matches_library_topk_on_tie_free_input(rng):
    # The page's recipe selects the top-2 of |w| per group of 4 along K; on
    # tie-free input torch.topk gives that set without needing a tie rule.
    n, k = 64, 512
    x = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32))
    xb = x.to(torch.bfloat16)
    bits = W.bf16_bits(xb)
    g = xb.float().abs().reshape(n, k // 4, 4)
    srt = torch.sort(g, dim=-1).values
    tie_free = bool((srt[..., 1:] != srt[..., :-1]).all())
    if not tie_free:
        # remove the groups with ties from the comparison
        keep_rows = (srt[..., 1:] != srt[..., :-1]).all(-1)
    else:
        keep_rows = torch.ones(n, k // 4, dtype=torch.bool)
    top = torch.topk(g, 2, dim=-1).indices
    lib_mask = torch.zeros_like(g, dtype=torch.bool).scatter_(-1, top, True)
    ours = torch.from_numpy(O.prune_mask(bits).reshape(n, k // 4, 4))
    assert torch.equal(ours[keep_rows], lib_mask[keep_rows])
    assert int(keep_rows.sum()) > 0.9 * keep_rows.numel()


def test_rejects_k_not_multiple_of_4():
    with pytest.raises(ValueError):
        O.prune_mask(np.zeros((2, 6), dtype=np.uint16))


def test_compress_layout_hand_example():
    # one row, 32 values = 8 groups = one metadata word
    vals = np.zeros((1, 32), dtype=np.float32)
    # group 0: keep positions 1, 3 ; group 1: keep 0, 2 ; group 2: ties -> 0, 1
    vals[0, 0:4] = [0.1, -5.0, 0.2, 4.0]
    vals[0, 4:8] = [7.0, 1.0, -7.5, 0.5]
    vals[0, 8:12] = [2.0, 2.0, 2.0, 2.0]
    vals[0, 12:16] = [0.0, 0.0, 0.0, 3.0]  # keep 0 (tie at zero, lower index) and 3
    bits = _bf16_bits_of(vals)
    v, meta = O.prune_compress(bits)
    assert v.shape == (1, 16) and meta.shape == (1, 1)
    f = O.bf16_to_f32(v)[0]
    assert list(f[:8]) == [-5.0, 4.0, 7.0, -7.5, 2.0, 2.0, 0.0, 3.0]
    nibs = [(int(meta[0, 0]) >> (4 * g)) & 0xF for g in range(8)]
    assert nibs[0] == (1 | 3 << 2)
    assert nibs[1] == (0 | 2 << 2)
    assert nibs[2] == (0 | 1 << 2)
    assert nibs[3] == (0 | 3 << 2)
    assert all(nb == (0 | 1 << 2) for nb in nibs[4:])  # all-zero groups keep 0, 1


@pytest.mark.parametrize("shape", [(1, 32), (3, 64), (17, 352), (64, 1024)])
def test_round_trips(rng, shape):
    n, k = shape
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    bits = W.bf16_bits(x.to(torch.bfloat16))
    mask = O.prune_mask(bits)
    v, meta = O.compress(bits, mask)
    assert v.shape == (n, k // 2) and meta.shape == (n, k // 32)
    pruned = O.apply_mask(bits, mask)
    assert np.array_equal(O.decompress(v, meta, k), pruned)
    assert np.array_equal(O.mask_from_meta(meta, k), mask)
    v2, meta2 = O.compress(O.decompress(v, meta, k), O.mask_from_meta(meta, k))
    assert np.array_equal(v2, v) and np.array_equal(meta2, meta)
    nib = (meta[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    assert set(np.unique(nib).tolist()) <= {4, 8, 9, 12, 13, 14}


def test_decompress_works_on_fp8_codes(rng):
    codes = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)
    codes[codes == 0x7F] = 1
    bits = np.zeros((5, 128), dtype=np.uint16)
    mask = np.zeros((5, 128), dtype=bool)
    # choose random valid masks
    pairs = list(itertools.combinations(range(4), 2))
    for r in range(5):
        for g in range(32):
            i, j = pairs[rng.integers(0, 6)]
            mask[r, 4 * g + i] = mask[r, 4 * g + j] = True
    dense = np.zeros((5, 128), dtype=np.uint8)
    dense[mask] = codes.reshape(-1)
    v, meta = O.compress(dense, mask)
    assert np.array_equal(v, codes)
    assert np.array_equal(O.decompress(v, meta, 128), dense)
    del bits


def test_brute_force_on_workload_rows():
    # a slice of the tiny workload's weight, checked group by group
    _, w = W.tiny()
    bits = W.bf16_bits(w)[:8]
    mask = O.prune_mask(bits)
    mags = (bits & 0x7FFF).astype(np.int64)
    for r in range(8):
        for g in range(64):
            a = mags[r, 4 * g:4 * g + 4].tolist()
            assert tuple(np.nonzero(mask[r, 4 * g:4 * g + 4])[0].tolist()) == _brute_keep(a)


def test_meta_storage_order_hand_examples():
    # meta[r, w] = 16 r + w; blocks of 4 words, rows one after another per block
    m = (16 * np.arange(2)[:, None] + np.arange(5)[None, :]).astype(np.uint32)   # K = 160
    assert O.store_meta(m).tolist() == [0, 1, 2, 3, 16, 17, 18, 19, 4, 20]
    m = (16 * np.arange(3)[:, None] + np.arange(8)[None, :]).astype(np.uint32)   # K = 256
    assert O.store_meta(m).tolist() == [0, 1, 2, 3, 16, 17, 18, 19, 32, 33, 34, 35,
                                        4, 5, 6, 7, 20, 21, 22, 23, 36, 37, 38, 39]
    m = (16 * np.arange(2)[:, None] + np.arange(3)[None, :]).astype(np.uint32)   # K = 96: one short block
    assert O.store_meta(m).tolist() == [0, 1, 2, 16, 17, 18]


@pytest.mark.parametrize("n,k", [(1, 32), (1, 4096), (5, 96), (7, 160), (33, 1024), (4, 1120)])
def test_meta_storage_order_is_a_permutation(n, k):
    idx = O.meta_word_index(n, k)
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(n * (k // 32)))
    m = np.random.default_rng(n * k).integers(0, 2**32, size=(n, k // 32), dtype=np.uint64).astype(np.uint32)
    s = O.store_meta(m)
    assert np.array_equal(O.load_meta(s, n, k), m)
    if n == 1 or k <= 128:
        assert np.array_equal(s, m.reshape(-1))   # one row, or one block: row order
    if k % 128 == 0:
        # block b of row r is the 16 bytes at (b * n + r) * 4 words
        b = np.arange(k // 128)
        for r in (0, n - 1):
            assert np.array_equal(s.reshape(k // 128, n, 4)[b, r].reshape(-1), m[r])
