"""GPU parity of sp24_gemm (and the dense baseline) against the oracle.

Bar: every output within |y - ref| <= 8e-3 |ref| + 1e-4 sum_k |x_k w_k| (y the
BF16 output, ref the float64 product of the oracle's own compressed and
quantised operands), and all intermediate codes bit-exact.  Shapes span
several tiles, ragged m and n, every K tail (K mod 512 in {0,128,256,384}),
the K split, and the full workload sizes (sampled where the oracle would take
too long).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (GpuWeight, OracleWeight, announce, assert_within_tolerance, bits, codes,
                         f32, f32_bits, gpu_x, need_sp, oracle_ref, oracle_x, u32)
from gpu_helpers import full_case as _full_case
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def test_tiny_workload_bf16():
    x, w = W.tiny()
    _full_case(x, w, False, "tiny")


def test_tiny_workload_fp8():
    x, w = W.tiny()
    _full_case(x, w, True, "tiny")


SHAPES = [(1, 16, 128), (3, 17, 256), (16, 64, 384), (17, 100, 640), (33, 48, 1152),
          (64, 256, 2048), (65, 40, 512), (100, 33, 1408), (8, 32, 16384), (129, 80, 896),
          # LDS-tiled kernel: ragged tiles in m and n, several K steps
          (1000, 8200, 640), (2048, 8192, 1024), (777, 32784, 256),
          # ... and n not a multiple of 8 (the epilogue's per-element tail)
          (600, 32771, 384), (1111, 8198, 256)]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_random_shapes(m, n, k, fp8):
    seed = m * 7919 + n * 31 + k
    x = W.randn_bf16((m, k), seed=seed)
    w = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
    _full_case(x, w, fp8, "random %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("m", [1, 16, 64])
def test_decode_up_projection(m, fp8):
    _full_case(W.up_x(m), W.up_weight(), fp8, "up M=%d" % m)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("m", [1, 16, 64])
def test_decode_down_projection(m, fp8):
    _full_case(W.down_x(m), W.down_weight(), fp8, "down M=%d" % m)


@pytest.mark.parametrize("fp8", [False, True])
def test_dense_baseline(fp8):
    _full_case(W.up_x(16), W.up_weight()[:1024], fp8, "dense up slice", dense=True)
    x = W.randn_bf16((33, 640), seed=5)
    w = W.randn_bf16((100, 640), seed=6, std=0.02)
    _full_case(x, w, fp8, "dense ragged", dense=True)
    x = W.randn_bf16((1000, 640), seed=7)
    w = W.randn_bf16((8200, 640), seed=8, std=0.02)
    _full_case(x, w, fp8, "dense tiled ragged", dense=True)


def test_bitwise_reproducible_and_split_k():
    sp = need_sp()
    for m, n, k in ((16, 1024, 16384), (8, 32, 16384)):
        pl = sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)
        assert pl["split_k"] > 1
        x = W.randn_bf16((m, k), seed=m + k)
        w = W.randn_bf16((n, k), seed=n + k, std=0.02)
        y1, _ = _full_case(x, w, True, "split-K %dx%dx%d" % (m, n, k))
        xq, xs = gpu_x(x, True)
        gw = GpuWeight(w, True)
        y2 = sp.gemm(xq, gw.qvalues, gw.meta, x_scale=xs, w_scale=gw.scale)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def _sampled_case(x_cpu, w_cpu, fp8, what, n_rows=512, n_tokens=None, seed=0):
    """Full-size GPU run; the oracle checks a random sample of W rows (and tokens)."""
    sp = need_sp()
    announce("gemm sampled", what, "fp8" if fp8 else "bf16", tuple(x_cpu.shape), tuple(w_cpu.shape))
    gw = GpuWeight(w_cpu, fp8)
    xq, xs = gpu_x(x_cpu, fp8)
    y = sp.gemm(xq, gw.qvalues, gw.meta, x_scale=xs, w_scale=gw.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    n, m = w_cpu.shape[0], x_cpu.shape[0]
    rows = np.sort(rng.choice(n, size=min(n_rows, n), replace=False))
    rows = np.unique(np.concatenate([rows, [0, n - 1]]))
    toks = np.arange(m) if n_tokens is None else np.unique(np.concatenate(
        [np.sort(rng.choice(m, size=n_tokens, replace=False)), [0, m - 1]]))
    wb = W.bf16_bits(w_cpu)
    ow = OracleWeight(wb, fp8, rows=rows)
    xb = W.bf16_bits(x_cpu)
    if fp8:
        oxs = O.fp8_scale(xb)                       # per-tensor: from every value
        oxq, _ = O.quant_fp8(xb[toks], scale=oxs)   # then the sampled tokens' codes
        assert f32_bits(f32(xs)) == f32_bits(oxs)
        assert f32_bits(f32(gw.scale)) == f32_bits(ow.scale)
        gq = codes(gw.qvalues)[rows]
        assert np.array_equal(gq, ow.qvalues)
        assert np.array_equal(codes(xq)[toks], oxq)
    else:
        oxq, oxs = xb[toks], None
        assert np.array_equal(bits(gw.values)[rows], ow.values)
    assert np.array_equal(O.load_meta(u32(gw.meta), n, gw.k, rows), ow.meta)
    ref, mag = oracle_ref(oxq, oxs, ow)
    yb = bits(y)[np.ix_(toks, rows)]
    assert_within_tolerance(yb, ref, mag, what)


def test_prefill_sampled_fp8():
    _sampled_case(W.prefill_x(), W.prefill_weight(), True, "prefill", n_rows=256, n_tokens=256)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layer", [0, 31])
def test_layer_sweep_sampled(layer, fp8):
    for proj, (name, k, n) in enumerate(W.LAYER_PROJS):
        _sampled_case(W.layer_x(k), W.layer_weight(layer, proj), fp8, "layer %d %s" % (layer, name),
                      n_rows=256, seed=layer * 4 + proj)
