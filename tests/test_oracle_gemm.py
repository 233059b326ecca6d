"""Pins for the oracle's reference product Y = X . W^T over 2:4-pruned weights.

The product is the linear/FFN projection the cookbook page ("Deploying 2:4
Sparsity with FP8 on Hopper") prunes (pipeline step 2: groups along K of the
[out, in] weight).  The oracle decompresses and multiplies in float64; these
tests check it against a pure-Python triple loop that reads the keep-mask
directly (never the compressed form), plus closed-form special cases.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O


def _triple_loop(x, w, mask):
    m, k = len(x), len(x[0])
    n = len(w)
    out = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                if mask[j][kk]:
                    acc += float(x[i][kk]) * float(w[j][kk])
            out[i][j] = acc
    return np.array(out)


@pytest.mark.parametrize("m,n,k", [(3, 5, 32), (2, 7, 64), (1, 3, 96)])
def test_bf16_product_matches_triple_loop(rng, m, n, k):
    x = W.bf16_bits(torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16))
    w = W.bf16_bits(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.bfloat16))
    mask = O.prune_mask(w)
    v, meta = O.compress(w, mask)
    xh, wh = O.sparse_operands_bf16(x, v, meta, k)
    ref, mag = O.gemm_ref(xh, wh)
    brute = _triple_loop(O.bf16_to_f64(x).tolist(), O.bf16_to_f64(w).tolist(), mask.tolist())
    assert ref.shape == (m, n)
    np.testing.assert_allclose(ref, brute, rtol=1e-12, atol=1e-12)
    brute_mag = _triple_loop(np.abs(O.bf16_to_f64(x)).tolist(), np.abs(O.bf16_to_f64(w)).tolist(),
                             mask.tolist())
    np.testing.assert_allclose(mag, brute_mag, rtol=1e-12, atol=1e-12)


def test_fp8_product_matches_triple_loop(rng):
    m, n, k = 3, 4, 64
    x = W.bf16_bits(torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16))
    w = W.bf16_bits(torch.from_numpy((0.02 * rng.standard_normal((n, k))).astype(np.float32)).to(torch.bfloat16))
    mask = O.prune_mask(w)
    v, meta = O.compress(w, mask)
    xq, sx = O.quant_fp8(x)
    vq, sw = O.quant_fp8(v)
    xh, wh = O.sparse_operands_fp8(xq, sx, vq, meta, sw, k)
    ref, _ = O.gemm_ref(xh, wh)
    # triple loop over the dense pruned weight quantised element by element
    wq_dense = np.zeros((n, k), dtype=np.uint8)
    wq_dense[mask] = O.e4m3_encode(O.bf16_to_f32(w[mask]) / sw)
    xdq = (O.e4m3_decode(xq) * np.float64(sx)).tolist()
    wdq = (O.e4m3_decode(wq_dense) * np.float64(sw)).tolist()
    np.testing.assert_allclose(ref, _triple_loop(xdq, wdq, mask.tolist()), rtol=1e-12, atol=1e-15)


def test_one_hot_rows_pick_columns_of_w(rng):
    n, k = 6, 64
    w = W.bf16_bits(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.bfloat16))
    v, meta = O.prune_compress(w)
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = 0x3F80  # bf16 1.0
    xh, wh = O.sparse_operands_bf16(x, v, meta, k)
    ref, _ = O.gemm_ref(xh, wh)
    pruned = O.bf16_to_f64(O.apply_mask(w, O.prune_mask(w)))
    assert np.array_equal(ref, pruned.T)   # row kk of Y is column kk of the pruned W


def test_all_ones_gives_row_sums_over_kept(rng):
    n, k = 9, 128
    w = W.bf16_bits(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.bfloat16))
    mask = O.prune_mask(w)
    v, meta = O.compress(w, mask)
    x = np.full((2, k), 0x3F80, dtype=np.uint16)
    ref, mag = O.gemm_ref(*O.sparse_operands_bf16(x, v, meta, k))
    wf = O.bf16_to_f64(w)
    want = np.array([sum(wf[r, c] for c in range(k) if mask[r, c]) for r in range(n)])
    np.testing.assert_allclose(ref[0], want, rtol=1e-13)
    np.testing.assert_allclose(mag[1], np.abs(wf * mask).sum(1), rtol=1e-13)


def test_sum_over_kept_equals_masked_dense(rng):
    m, n, k = 4, 8, 256
    x = W.bf16_bits(torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16))
    w = W.bf16_bits(torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.bfloat16))
    mask = O.prune_mask(w)
    v, meta = O.compress(w, mask)
    ref, _ = O.gemm_ref(*O.sparse_operands_bf16(x, v, meta, k))
    dense = O.bf16_to_f64(x) @ (O.bf16_to_f64(w) * mask).T
    np.testing.assert_allclose(ref, dense, rtol=1e-12, atol=1e-12)
    # and not the unpruned product (a dropped mask would pass the test above trivially)
    full = O.bf16_to_f64(x) @ O.bf16_to_f64(w).T
    assert not np.allclose(ref, full, rtol=1e-3)


def test_tolerance_rule():
    ref = np.array([1.0, -2.0, 0.0])
    mag = np.array([10.0, 10.0, 10.0])
    assert O.within_tolerance(np.array([1.008, -2.0, 0.001]), ref, mag).all()
    assert not O.within_tolerance(np.array([1.0 + 0.0091, -2.0, 0.0]), ref, mag)[0]
    assert not O.within_tolerance(np.array([1.0, -2.0, 0.0011]), ref, mag)[2]
