"""Seeded input generators: deterministic, right shapes and distributions."""
import hashlib

import numpy as np
import torch

import workloads as W


def _h(t):
    return hashlib.sha256(W.bf16_bits(t).tobytes()).hexdigest()


def test_deterministic():
    a, b = W.tiny(), W.tiny()
    assert _h(a[0]) == _h(b[0]) and _h(a[1]) == _h(b[1])
    assert _h(W.up_x(16)) == _h(W.up_x(16))
    assert _h(W.up_x(16)) != _h(W.up_x(64)[:16])


def test_shapes_and_dtypes():
    x, w = W.tiny()
    assert x.shape == (8, 256) and w.shape == (256, 256)
    assert x.dtype == w.dtype == torch.bfloat16
    assert W.up_x(1).shape == (1, 4096)
    assert W.down_x(16).shape == (16, 14336)
    assert W.layer_x(4096).shape == (256, 4096) and W.layer_x(14336).shape == (256, 14336)


def test_distributions():
    _, w = W.tiny()
    assert abs(float(w.float().std()) - 0.02) < 0.001
    x = W.up_x(64).float()
    ch = W.up_outlier_channels()
    assert len(ch) == 41
    others = torch.ones(4096, dtype=torch.bool)
    others[ch] = False
    r = float(x[:, ch].std() / x[:, others].std())
    assert 17 < r < 23
    d = W.down_x(64).float()
    assert float(d.min()) > -0.3  # SiLU's minimum is about -0.278
    assert abs(float(d.mean()) - 0.207) < 0.02  # E[SiLU(Z)] for Z ~ N(0,1)


def test_bits_round_trip():
    x = W.randn_bf16((3, 5), seed=7)
    assert torch.equal(W.bits_to_bf16(W.bf16_bits(x)).view(3, 5), x)
    assert W.bf16_bits(x).dtype == np.uint16
