"""Pins of the oracle's INT8 quantisation (symmetric, per tensor):
s = fp32(amax / 127), q = clamp(round_half_even(fp32(v / s)), -127, 127)."""
import numpy as np
import torch

import workloads as W
from oracle import sp24_ref as O


def _bits(a):
    return W.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_amax_maps_to_127_and_scale_bits():
    x = _bits([[0.5, -254.0, 3.0, 0.0]])
    q, s = O.quant_int8(x)
    assert s == np.float32(254.0) / np.float32(127.0) == np.float32(2.0)
    assert q.tolist() == [[0, -127, 2, 0]]          # 0.25 -> 0, 1.5 -> 2 (ties to even)


def test_ties_go_to_even():
    # with s = 1 (static), x / s is exact: halves round to the even neighbour
    x = _bits([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 126.5])
    q, _ = O.quant_int8(x, scale=1.0)
    assert q.tolist() == [0, 2, 2, 0, -2, -2, 4, 126]


def test_static_scale_saturates_symmetrically():
    q, _ = O.quant_int8(_bits([1000.0, -1000.0, 127.4, -127.6]), scale=1.0)
    assert q.tolist() == [127, -127, 127, -127]    # never -128


def test_zero_tensor_and_dequant():
    q, s = O.quant_int8(np.zeros(16, dtype=np.uint16))
    assert s == 1.0 and not q.any()
    assert O.dequant_int8(np.array([-127, 0, 5], dtype=np.int8), 0.5).tolist() == [-63.5, 0.0, 2.5]


def test_random_matches_torch_round(rng):
    x = _bits(rng.standard_normal((5, 333)).astype(np.float32) * 7)
    q, s = O.quant_int8(x)
    # torch.round is half-to-even as well; an independent evaluation of the same definition
    t = torch.from_numpy(O.bf16_to_f32(x)) / torch.tensor(s)
    ref = torch.clamp(torch.round(t), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(q, ref)
    assert np.abs(q).max() == 127
    # dequantised values within half a step of the input, plus the float32 rounding of the
    # quotient x / s (|x / s| <= 127, relative error <= 2^-24) taken before the integer rounding
    assert np.all(np.abs(O.dequant_int8(q, s) - O.bf16_to_f64(x)) <= (0.5 + 127 * 2.0 ** -24) * s + 1e-12)


def test_rows_are_independent_and_one_row_is_per_tensor(rng):
    x = rng.standard_normal((4, 96)).astype(np.float32)
    x[1] *= 300.0                                    # an outlier row does not touch the others
    x[3] = 0.0                                       # a zero row gets scale 1 and zero codes
    xb = _bits(x)
    q, s = O.quant_int8_rows(xb)
    for m in range(4):
        qm, sm = O.quant_int8(xb[m])
        assert s[m] == sm and np.array_equal(q[m], qm)
    assert s[3] == 1.0 and not q[3].any()
    assert np.abs(q[[0, 1, 2]]).max(axis=1).tolist() == [127, 127, 127]


def test_int8_product_is_the_integer_product(rng):
    """The dequantised product equals sx * sw * (integer dot product), up to float64
    rounding of the dequantised terms (each (sx qx)(sw qw) needs up to 64 bits)."""
    k = 256
    x = _bits(rng.standard_normal((3, k)).astype(np.float32))
    w = _bits(rng.standard_normal((5, k)).astype(np.float32))
    vals, meta = O.prune_compress(w)
    wq, sw = O.quant_int8(vals)
    xq, sx = O.quant_int8(x)
    xh, wh = O.sparse_operands_int8(xq, sx, wq, meta, sw, k)
    ref, mag = O.gemm_ref(xh, wh)
    wd = O.decompress(wq, meta, k).astype(np.int64)
    exact = xq.astype(np.int64) @ wd.T                       # integer arithmetic
    want = np.float64(sx) * np.float64(sw) * exact.astype(np.float64)
    assert np.all(np.abs(ref - want) <= 1e-13 * mag)
    assert np.abs(exact).max() > 1000                        # a real sum, not a trivial one
    # the decompressed INT8 weight holds the kept codes at their positions and zeros elsewhere
    assert (np.count_nonzero(wd.reshape(5, -1, 4), axis=2) <= 2).all()
