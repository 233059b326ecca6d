"""Pins of the oracle's SlideSparse transform ("SlideSparse: Fast and Flexible
(2N-2):2N Structured Sparsity", technical summary, section 2): every
(2N-2):2N block fits N-1 overlapping 2:4 windows, the packed weight is 2:4,
lifting the activations keeps the product exact, and K grows by (2N-2)/N."""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O


@pytest.mark.parametrize("n_pat", [2, 3, 4, 5])
def test_every_block_of_at_most_2n_minus_2_nonzeros_fits(n_pat):
    blk = 2 * n_pat
    for mask in itertools.product([0, 1], repeat=blk):
        nnz = sum(mask)
        if nnz > blk - 2:
            continue
        owner = O.slide_windows(mask, n_pat)
        # every nonzero has a window that covers it, zeros have none, at most 2 per window
        for p in range(blk):
            if mask[p]:
                j = owner[p]
                assert 0 <= j <= n_pat - 2 and 2 * j <= p < 2 * j + 4, (mask, owner)
            else:
                assert owner[p] == -1
        for j in range(n_pat - 1):
            assert owner.count(j) <= 2


@pytest.mark.parametrize("n_pat", [3, 4])
def test_too_dense_blocks_are_rejected(n_pat):
    with pytest.raises(ValueError):
        O.slide_windows([1] * (2 * n_pat), n_pat)


def test_page_example_6_of_8():
    # 6 of 8 nonzero: 3 windows of 4 = 12 values, each window 2:4
    block = np.array([[1, 2, 3, 4, 5, 6, 0, 0]], dtype=np.int64)
    assert O.slide_pack(block, 4).tolist() == [[1, 2, 0, 0, 3, 4, 0, 0, 5, 6, 0, 0]]
    block = np.array([[1, 0, 2, 3, 4, 0, 5, 6]], dtype=np.int64)
    # window 0 must take position 0, then 2; window 1 must take 3, then 4; window 2 takes 6, 7
    assert O.slide_pack(block, 4).tolist() == [[1, 0, 2, 0, 0, 3, 4, 0, 0, 0, 5, 6]]
    assert O.slide_lift(np.arange(8)[None, :], 4).tolist() == [[0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7]]


@pytest.mark.parametrize("n_pat", [3, 4, 5])
def test_pack_and_lift_keep_the_product_exact(n_pat):
    rng = np.random.default_rng(n_pat)
    rows, k, m = 9, 2 * n_pat * 12, 5
    w = rng.integers(-50, 50, size=(rows, k))
    w = np.where(O.slide_prune_mask(W.bf16_bits(torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16)),
                                    n_pat), w, 0)
    x = rng.integers(-50, 50, size=(m, k))
    wp, xl = O.slide_pack(w, n_pat), O.slide_lift(x, n_pat)
    assert wp.shape == (rows, k * (2 * n_pat - 2) // n_pat) and xl.shape == (m, wp.shape[1])
    assert np.all((wp.reshape(rows, -1, 4) != 0).sum(-1) <= 2)       # 2:4 along K'
    assert np.array_equal(xl @ wp.T, x @ w.T)                         # exact integers
    assert np.count_nonzero(wp) == np.count_nonzero(w)                # nothing lost, nothing added


def test_prune_mask_6_of_8_by_brute_force():
    rng = np.random.default_rng(3)
    vals = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0], dtype=np.float32), size=(40, 64))
    bits = W.bf16_bits(torch.from_numpy(vals).to(torch.bfloat16))
    mask = O.slide_prune_mask(bits, 4)
    for r in range(40):
        for b in range(8):
            a = [abs(float(v)) for v in vals[r, 8 * b:8 * b + 8]]
            order = sorted(range(8), key=lambda i: (-a[i], i))   # largest first, lower index on ties
            keep = set(order[:6])
            assert [bool(mask[r, 8 * b + i]) for i in range(8)] == [i in keep for i in range(8)]


def test_lifted_activations_keep_per_token_scales():
    # every position of X appears in some window, so the row maximum and the codes carry over
    x = W.bf16_bits(W.randn_bf16((3, 64), seed=4))
    q, s = O.quant_fp8_rows(x)
    ql, sl = O.quant_fp8_rows(O.slide_lift(x, 4))
    assert np.array_equal(s, sl) and np.array_equal(ql, O.slide_lift(q, 4))
