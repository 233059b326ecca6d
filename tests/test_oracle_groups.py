"""Pins of the oracle's finer FP8 scales: one dynamic scale per group of consecutive
values of a row (per-group along K, per-channel as one group per row), and the float64
reference product with group scales.

The research-roadmap page ("La Densite Dynamique et les Noyaux Non Structures",
quantisation under extreme sparsity) asks for per-channel or per-group scales; every
group is quantised as the per-tensor recipe would quantise it alone.  Each pin is
chosen so that a plausible slip (a wrong group index, a transposed scale array, a scale
taken from the wrong slice, a group of compressed values not matching its K positions)
fails at least one of them."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O


def _bits(a):
    return W.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_hand_example():
    # row 0: group 0 holds 448 (its scale is 1, codes are the values' own E4M3 codes);
    # group 1 holds 0.25 as its maximum (scale 0.25 / 448, which maps 0.25 to 448 = 0x7E)
    # and a negative zero (code 0x80); row 1 is all zero (scales 1, codes 0)
    x = _bits([[448.0, 1.0, -2.0, 0.5, 0.25, 0.0, 0.0, -0.0],
               [0.0] * 8])
    q, s = O.quant_fp8_groups(x, 4)
    assert s.dtype == np.float32 and s.shape == (2, 2)
    assert s[0, 0] == np.float32(1.0)
    assert s[0, 1] == np.float32(0.25) / np.float32(448.0)
    assert s[1].tolist() == [1.0, 1.0]
    assert q[0].tolist() == [0x7E, 0x38, 0xC0, 0x30, 0x7E, 0x00, 0x00, 0x80]
    assert not q[1].any()


def test_each_group_is_the_per_tensor_recipe_on_its_own_slice(rng):
    x = _bits(rng.standard_normal((5, 384)).astype(np.float32) * rng.uniform(0.01, 50, (5, 1)).astype(np.float32))
    for group in (8, 32, 128, 384):
        q, s = O.quant_fp8_groups(x, group)
        assert q.shape == x.shape and s.shape == (5, 384 // group)
        for r in range(5):
            for g in range(384 // group):
                qg, sg = O.quant_fp8(x[r, g * group:(g + 1) * group])
                assert s[r, g] == sg and np.array_equal(q[r, g * group:(g + 1) * group], qg), (group, r, g)


def test_one_group_per_row_is_per_token(rng):
    x = _bits(rng.standard_normal((6, 256)).astype(np.float32) * 3)
    x[2] = 0
    q, s = O.quant_fp8_groups(x, 256)
    qr, sr = O.quant_fp8_rows(x)
    assert np.array_equal(q, qr) and np.array_equal(s[:, 0], sr)


def test_power_of_two_scaling_moves_only_that_groups_scale(rng):
    x = rng.uniform(-4, 4, (3, 512)).astype(np.float32)
    q0, s0 = O.quant_fp8_groups(_bits(x), 128)
    y = x.copy()
    y[1, 256:384] *= 8.0                         # exact in bfloat16 at these magnitudes
    q1, s1 = O.quant_fp8_groups(_bits(y), 128)
    assert np.array_equal(q0, q1)                # codes do not move
    expect = s0.copy()
    expect[1, 2] *= np.float32(8.0)
    assert np.array_equal(s1, expect)            # only scale (1, 2) moves, by exactly 8


def test_equal_group_maxima_reduce_to_one_scale_per_tensor(rng):
    x = rng.uniform(-1, 1, (4, 256)).astype(np.float32)
    x[:, ::64] = 3.0                             # every group of 64 holds the tensor's maximum
    xb = _bits(x)
    q, s = O.quant_fp8_groups(xb, 64)
    qt, st = O.quant_fp8(xb)
    assert np.all(s == st) and np.array_equal(q, qt)


def test_dequantised_values_are_within_half_a_step(rng):
    x = _bits(rng.standard_normal((3, 256)).astype(np.float32) * 10)
    q, s = O.quant_fp8_groups(x, 128)
    d = O.dequant_fp8_groups(q, s, 128)
    xv = O.bf16_to_f64(x)
    ss = np.repeat(s.astype(np.float64), 128, axis=1)
    # E4M3 keeps 3 mantissa bits: half a step is 2^-4 relative in the normal range and
    # 2^-10 * s below it; the group maximum maps to 448 and comes back within 2^-4
    assert np.all(np.abs(d - xv) <= np.abs(xv) * 2.0 ** -4 + ss * 2.0 ** -10 + 1e-30)


def test_weight_group_scales_from_compressed_values_equal_those_of_the_pruned_weight(rng):
    # the kept values of K positions [group*g, group*(g+1)) are compressed columns
    # [group/2*g, group/2*(g+1)); dropped values are zeros and cannot raise a maximum
    w = _bits(rng.standard_normal((7, 512)).astype(np.float32) * 0.02)
    values, meta = O.prune_compress(w)
    pruned = O.decompress(values, meta, 512)
    for group in (128, 256, 512):
        assert np.array_equal(O.fp8_group_scales(values, group // 2), O.fp8_group_scales(pruned, group))


@pytest.mark.parametrize("group", [128, 256])
def test_reference_product_equals_a_triple_loop_over_the_mask(group, rng):
    m, n, k = 3, 5, 512
    xb = _bits(rng.standard_normal((m, k)).astype(np.float32) * rng.uniform(0.1, 20, (m, 1)).astype(np.float32))
    wb = _bits(rng.standard_normal((n, k)).astype(np.float32) * 0.02)
    values, meta = O.prune_compress(wb)
    wq, w_scales = O.quant_fp8_groups(values, group // 2)
    xq, x_scales = O.quant_fp8_groups(xb, group)
    ref, mag = O.gemm_ref(*O.sparse_operands_fp8_groups(xq, x_scales, wq, meta, w_scales, k, group))
    # the keep mask straight from the pruning rule (not through compress/decompress): the
    # j-th kept value of row r sits at the j-th kept position
    mask = O.prune_mask(wb)
    dec = O.e4m3_decode
    for r in range(m):
        for c in range(n):
            kept = np.nonzero(mask[c])[0]
            tot = totabs = 0.0
            for g in range(k // group):
                part = 0.0
                for j, kk in enumerate(kept):
                    if kk // group != g:
                        continue
                    assert j // (group // 2) == g   # its compressed column lies in the same group
                    part += float(dec(xq[r, kk])) * float(dec(wq[c, j]))
                    totabs += abs(float(x_scales[r, g]) * float(dec(xq[r, kk])) *
                                  float(w_scales[c, g]) * float(dec(wq[c, j])))
                tot += float(x_scales[r, g]) * float(w_scales[c, g]) * part
            assert abs(ref[r, c] - tot) <= 1e-12 * max(1.0, abs(tot)), (r, c)
            assert abs(mag[r, c] - totabs) <= 1e-12 * max(1.0, totabs), (r, c)


def test_one_group_product_equals_the_per_row_reference(rng):
    # group = K: per-token X scales times per-output-channel W scales; with one channel
    # scale shared by every row it is the per-token path with a per-tensor W scale
    m, n, k = 4, 6, 256
    xb = _bits(rng.standard_normal((m, k)).astype(np.float32))
    wb = _bits(rng.standard_normal((n, k)).astype(np.float32) * 0.02)
    values, meta = O.prune_compress(wb)
    xq, xs = O.quant_fp8_rows(xb)
    wq, sw = O.quant_fp8(values)
    ref_rows, _ = O.gemm_ref(*O.sparse_operands_fp8_rows(xq, xs, wq, meta, sw, k))
    ws = np.full((n, 1), sw, dtype=np.float32)
    ref_g, _ = O.gemm_ref(*O.sparse_operands_fp8_groups(xq, xs[:, None], wq, meta, ws, k, k))
    assert np.allclose(ref_g, ref_rows, rtol=1e-14, atol=0)
