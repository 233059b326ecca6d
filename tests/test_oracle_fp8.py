"""Pins for the oracle's FP8-E4M3 encoder, decoder and per-tensor scaling.

Per-tensor dynamic scaling follows the cookbook page ("Deploying 2:4 Sparsity
with FP8 on Hopper"), pipeline steps 3 and 6, and the clip-max advice in
"Troubleshooting quick hits".  The E4M3 format itself is pinned against the
OCP OFP8 specification (tests/golden/e4m3_ocp_points.txt) and PyTorch's
independent ``float8_e4m3fn`` implementation.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_cast(t):
    """PyTorch's float32 -> e4m3fn cast after an explicit clamp (torch does not saturate)."""
    tt = torch.from_numpy(np.asarray(t, dtype=np.float32))
    return torch.clamp(tt, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_ocp_points():
    with open(os.path.join(GOLDEN, "e4m3_ocp_points.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    tab = O.e4m3_value_table()
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        if np.isnan(val):
            assert np.isnan(tab[code])
        else:
            assert tab[code] == val and np.signbit(tab[code]) == np.signbit(val)
    assert np.isnan(tab).sum() == 2
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)            # codes 0..0x7E ascending
    assert np.array_equal(tab[0x80:0xFF], -pos)  # sign symmetry


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    fin = ~np.isnan(ours)
    assert np.array_equal(lib[fin], ours[fin])


def test_encode_exact_values_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def _neighbours(x):
    x = np.asarray(x, dtype=np.float32)
    return np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])


def test_encode_ties_and_neighbours_match_torch():
    pos = O.e4m3_value_table()[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact midpoints (all fp32-exact)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    pts = _neighbours(np.concatenate([mids, pos.astype(np.float32), [464.0, 480.0, 500.0, 1e6, 3.0e38]]))
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(O.e4m3_encode(pts), _torch_cast(pts))


def test_encode_random_matches_torch(rng):
    # log-uniform magnitudes over the whole fp32 range, both signs
    e = rng.uniform(-150, 128, size=200_000)
    x = (np.sign(rng.standard_normal(e.size)) * 2.0 ** e).astype(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(O.e4m3_encode(x), _torch_cast(x))
    y = rng.uniform(-460, 460, size=200_000).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(y), _torch_cast(y))


def test_encode_known_points():
    # values observed with PyTorch's cast and implied by the OCP definition
    pts = [(448.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),
           (1.5 * 2.0 ** -10, 0x01), (3 * 2.0 ** -10, 0x02), (17.0, 0x58), (18.0, 0x59),
           (19.0, 0x5A), (-0.0, 0x80), (0.0, 0x00), (-1.0, 0xB8), (1e30, 0x7E), (-1e30, 0xFE)]
    got = O.e4m3_encode(np.array([p[0] for p in pts], dtype=np.float32))
    assert [int(c) for c in got] == [p[1] for p in pts]


def test_encode_rejects_nan():
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([np.nan], dtype=np.float32))


def test_dynamic_scale_bits_and_amax_code(rng):
    x = torch.from_numpy(rng.standard_normal((7, 300)).astype(np.float32)) * 3
    bits = W.bf16_bits(x.to(torch.bfloat16))
    codes, s = O.quant_fp8(bits)
    amax = np.abs(O.bf16_to_f32(bits)).max()
    assert s.dtype == np.float32
    assert s == np.float32(np.float32(amax) / np.float32(448.0))
    # the float64 quotient rounded once to float32 is the same number
    assert s == np.float32(np.float64(amax) / 448.0)
    at = np.abs(O.bf16_to_f32(bits)) == amax
    assert np.all((codes[at] & 0x7F) == 0x7E)
    assert np.all((codes & 0x7F) <= 0x7E)   # dynamic mode never needs the clamp
    # decoding then multiplying by s recovers every value within half an e4m3 step
    deq = O.dequant_fp8(codes, s)
    err = np.abs(deq - O.bf16_to_f64(bits))
    assert np.all(err <= np.abs(O.bf16_to_f64(bits)) * 2.0 ** -4 + s * 2.0 ** -10 * 1.0000001)


def test_zero_tensor_scale_is_one():
    codes, s = O.quant_fp8(np.zeros(64, dtype=np.uint16))
    assert s == np.float32(1.0) and np.all(codes == 0)
    codes, s = O.quant_fp8(np.full(64, 0x8000, dtype=np.uint16))   # all -0
    assert s == np.float32(1.0) and np.all(codes == 0x80)


def test_static_scale_saturates():
    vals = torch.tensor([1.0, -1.0, 1000.0, -1000.0, 0.3], dtype=torch.float32).to(torch.bfloat16)
    codes, s = O.quant_fp8(W.bf16_bits(vals), scale=np.float32(0.5))
    assert s == np.float32(0.5)
    assert [int(c) for c in codes] == [0x40, 0xC0, 0x7E, 0xFE, int(_torch_cast([0.3 / 0.5])[0])]


def test_division_not_reciprocal():
    # v / s and v * (1/s) differ in float32 for some v; the oracle must divide.
    s = np.float32(3.0) / np.float32(448.0)
    v = np.arange(1, 20000, dtype=np.float32) * np.float32(0.001)
    bits = W.bf16_bits(torch.from_numpy(v).to(torch.bfloat16))
    vf = O.bf16_to_f32(bits)
    codes, _ = O.quant_fp8(bits, scale=s)
    assert np.array_equal(codes, O.e4m3_encode(vf / s))
    assert np.array_equal(codes, _torch_cast(vf / s))


def test_scale_after_pruning_equals_before():
    # recalibration after pruning: the group maximum survives pruning, so the
    # per-tensor amax (and the scale) of the pruned weight equal the dense one
    _, w = W.tiny()
    bits = W.bf16_bits(w)
    v, meta = O.prune_compress(bits)
    assert O.fp8_scale(v) == O.fp8_scale(bits)


# ---------------------------------------------------------------- per-row (per-token) scales

def _bits(a):
    return W.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_rows_single_value_maps_to_448():
    # row m holds one nonzero value v_m; its scale is |v_m| / 448 and v_m becomes +-448 (0x7E / 0xFE)
    x = np.zeros((3, 64), dtype=np.float32)
    x[0, 5], x[1, 63], x[2, 0] = 3.5, -0.0078125, 1000.0
    codes, s = O.quant_fp8_rows(_bits(x))
    assert s.shape == (3,) and s.dtype == np.float32
    assert s.tolist() == [np.float32(3.5) / np.float32(448), np.float32(0.0078125) / np.float32(448),
                          np.float32(1000) / np.float32(448)]
    assert codes[0, 5] == 0x7E and codes[1, 63] == 0xFE and codes[2, 0] == 0x7E
    mask = np.zeros_like(codes, dtype=bool)
    mask[0, 5] = mask[1, 63] = mask[2, 0] = True
    assert np.all(codes[~mask] == 0)


def test_rows_are_independent_of_each_other(rng):
    # an outlier row must not change the other rows' codes or scales (a per-tensor or
    # per-column scale would); each row matches torch's cast of that row over its own amax
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[2] *= 1000.0
    bits = _bits(x)
    codes, s = O.quant_fp8_rows(bits)
    xf = O.bf16_to_f32(bits)
    for m in range(4):
        amax = max(abs(float(v)) for v in xf[m])
        assert s[m] == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.array_equal(codes[m], _torch_cast(xf[m] / s[m]))
    # rows 0, 1, 3 are unchanged without the outlier row
    keep = [0, 1, 3]
    c2, s2 = O.quant_fp8_rows(bits[keep])
    assert np.array_equal(c2, codes[keep]) and np.array_equal(s2, s[keep])


def test_rows_power_of_two_scaling_changes_only_the_scale(rng):
    x = rng.standard_normal((1, 512)).astype(np.float32)
    rows = np.concatenate([x, x * 2.0 ** 7, x * 2.0 ** -5])   # exact in bf16
    codes, s = O.quant_fp8_rows(_bits(rows))
    assert np.array_equal(codes[0], codes[1]) and np.array_equal(codes[0], codes[2])
    assert s[1] == s[0] * np.float32(2.0 ** 7) and s[2] == s[0] * np.float32(2.0 ** -5)


def test_rows_reduce_to_per_tensor_for_one_row_and_zero_rows(rng):
    x = _bits(rng.standard_normal((1, 300)).astype(np.float32))
    c1, s1 = O.quant_fp8_rows(x)
    c0, s0 = O.quant_fp8(x)
    assert np.array_equal(c1, c0) and s1[0] == s0
    z = np.zeros((2, 64), dtype=np.uint16)
    cz, sz = O.quant_fp8_rows(z)
    assert np.all(sz == 1.0) and np.all(cz == 0)


def test_dequant_rows_by_hand():
    codes = np.array([[0x38, 0xB8, 0x00], [0x40, 0x7E, 0x01]], dtype=np.uint8)   # 1, -1, 0 ; 2, 448, 2^-9
    out = O.dequant_fp8_rows(codes, np.array([2.0, 0.5], dtype=np.float32))
    assert out.tolist() == [[2.0, -2.0, 0.0], [1.0, 224.0, 2.0 ** -10]]
