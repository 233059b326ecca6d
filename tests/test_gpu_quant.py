"""GPU parity of sp24_quant_fp8 against the oracle: E4M3 codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, announce, codes, f32, f32_bits, need_sp
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7FFF) < 0x7F80
    return b[finite]


def _gpu_static(x_bits, scale):
    sp = need_sp()
    x = W.bits_to_bf16(x_bits).to(DEV)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    q, s2 = sp.quant_fp8(x, scale=s)
    torch.cuda.synchronize()
    assert f32_bits(f32(s2)) == f32_bits(scale)   # static mode never writes the scale
    return codes(q)


def test_every_bf16_pattern_with_many_scales():
    xb = _all_finite_bf16()
    rng = np.random.default_rng(11)
    scales = [1.0, 0.5, 2.0 ** -20, 2.0 ** 20, 3.0 / 448.0, 1.0 / 448.0, 2.0 ** -126, 2.0 ** 100]
    scales += list(2.0 ** rng.uniform(-30, 30, size=24))
    for s in scales:
        s = np.float32(s)
        announce("quant static all bf16, scale", float(s))
        want, _ = O.quant_fp8(xb, scale=s)
        got = _gpu_static(xb, s)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "scale %r: %d codes differ, first x bits %#06x got %#04x want %#04x" % (
            float(s), bad.size, int(xb[bad[0]]), int(got[bad[0]]), int(want[bad[0]]))


def _dynamic(x_cpu, what):
    announce("quant dynamic", what, x_cpu.numel())
    sp = need_sp()
    q, s = sp.quant_fp8(x_cpu.to(DEV))
    torch.cuda.synchronize()
    xb = W.bf16_bits(x_cpu).reshape(-1)
    want, ws = O.quant_fp8(xb)
    assert f32_bits(f32(s)) == f32_bits(ws), "%s: scale %r vs %r" % (what, float(f32(s)), float(ws))
    got = codes(q).reshape(-1)
    assert np.array_equal(got, want), "%s: %d codes differ" % (what, int((got != want).sum()))


def test_dynamic_tiny():
    x, w = W.tiny()
    _dynamic(x, "tiny x")
    _dynamic(w, "tiny w")


@pytest.mark.parametrize("m", [1, 16, 64])
def test_dynamic_decode_activations(m):
    _dynamic(W.up_x(m), "up x")
    _dynamic(W.down_x(m), "down x")


@pytest.mark.parametrize("count", [1, 7, 8, 4095, 16391, 16392, 32768, 65543, 65544, 100003, 131072,
                                   131073, 1 << 20, (1 << 22) + 5])
def test_dynamic_sizes_and_tails(count):
    _dynamic(W.randn_bf16((count,), seed=count % 1000 + 1, std=3.0), "count")


def test_dynamic_full_weight_values():
    sp = need_sp()
    announce("quant weight values")
    v, _ = sp.prune_compress(W.up_weight().to(DEV))
    q, s = sp.quant_fp8(v)
    torch.cuda.synchronize()
    vb = W.bf16_bits(v.cpu()).reshape(-1)
    want, ws = O.quant_fp8(vb)
    assert f32_bits(f32(s)) == f32_bits(ws)
    assert np.array_equal(codes(q).reshape(-1), want)


def test_zero_and_negative_zero_tensors():
    for fill, code in ((0x0000, 0x00), (0x8000, 0x80)):
        for count in (100, 50000):
            xb = np.full(count, fill, dtype=np.uint16)
            announce("quant zero", hex(fill), count)
            q, s = need_sp().quant_fp8(W.bits_to_bf16(xb).to(DEV))
            torch.cuda.synchronize()
            assert f32(s) == np.float32(1.0)
            assert np.all(codes(q) == code)


def test_static_saturation():
    xb = W.bf16_bits(torch.tensor([1.0, -1.0, 300.0, -300.0, 1e30, -1e30, 0.01], dtype=torch.float32)
                     .to(torch.bfloat16))
    got = _gpu_static(xb, np.float32(0.5))
    want, _ = O.quant_fp8(xb, scale=np.float32(0.5))
    assert np.array_equal(got, want)
    assert list(got[2:6]) == [0x7E, 0xFE, 0x7E, 0xFE]


def _keys_spanning_the_divisor_routes():
    # largest magnitudes around the key 0x2000 (2^-63) below which the quantisers
    # divide, the extremes, and a spread of ordinary ones
    keys = [0x0001, 0x0080, 0x1FFF, 0x2000, 0x2001, 0x3F80, 0x43E0, 0x4380, 0x7F7F, 0x7F7E]
    keys += [int(k) for k in np.random.default_rng(5).integers(0x2000, 0x7F7F, size=22)]
    return keys


@pytest.mark.parametrize("dt", ["fp8", "int8"])
def test_dynamic_every_pattern_below_each_maximum(dt):
    """Dynamic per-tensor scales on every bf16 pattern of magnitude <= amax, for maxima
    on both sides of the key where the quantisers switch from the IEEE division to the
    reciprocal with one exact-residual correction: codes and scale bit-exact."""
    sp = need_sp()
    quant, oquant = (sp.quant_fp8, O.quant_fp8) if dt == "fp8" else (sp.quant_int8, O.quant_int8)
    b = np.arange(65536, dtype=np.uint32)
    for key in _keys_spanning_the_divisor_routes():
        xb = b[(b & 0x7FFF) <= key].astype(np.uint16)
        announce("quant dynamic every pattern below key", dt, hex(key), xb.size)
        x = W.bits_to_bf16(xb).to(DEV)
        q, s = quant(x)
        torch.cuda.synchronize()
        want, ws = oquant(xb)
        want = want.view(np.uint8)
        assert f32_bits(f32(s)) == f32_bits(ws), "key %#06x: scale differs" % key
        got = codes(q)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "key %#06x: %d codes differ, first x bits %#06x got %#04x want %#04x" % (
            key, bad.size, int(xb[bad[0]]), int(got[bad[0]]), int(want[bad[0]]))
