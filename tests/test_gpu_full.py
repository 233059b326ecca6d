"""Full-size parity, nothing sampled: the prefill GEMM (M=8192, K=8192, N=28672) and every
projection of layers 0, 15 and 31 of the layer sweep (M=256), FP8 with per-tensor scales.

Every kept value, metadata word, weight and activation code and both scales are compared
bit for bit with the oracle, and every output element against the oracle's float64
product within |y - ref| <= 8e-3 |ref| + 1e-4 sum_k |x_k w_k| (the prefill product in
blocks of 1024 tokens to bound host memory).  Slow: the oracle prunes and quantises 235 M
prefill weights and 218 M weights per layer on the host."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, announce, assert_within_tolerance, bits, codes, f32, f32_bits, need_sp, u32
from oracle import sp24_ref as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _gpu_side(x_cpu, w_cpu):
    """prune + compress + quantise W, quantise X and multiply on the GPU; everything back
    on the host (values bits, stored metadata, codes, scales, output bits)."""
    sp = need_sp()
    w = w_cpu.to(DEV)
    values, meta = sp.prune_compress(w)
    del w
    qv, sw = sp.quant_fp8(values)
    xq, sx = sp.quant_fp8(x_cpu.to(DEV))
    y = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    out = dict(values=bits(values), meta=u32(meta), qv=codes(qv), sw=f32(sw), xq=codes(xq), sx=f32(sx), y=bits(y))
    del values, meta, qv, xq, y
    torch.cuda.empty_cache()
    return out


def _check(x_cpu, w_cpu, what, block=1024):
    n, k = w_cpu.shape
    m = x_cpu.shape[0]
    announce("full-size", what, m, n, k)
    g = _gpu_side(x_cpu, w_cpu)
    wb, xb = W.bf16_bits(w_cpu), W.bf16_bits(x_cpu)
    ov, om = O.prune_compress(wb)
    assert np.array_equal(g["values"], ov), "%s: kept values differ" % what
    assert np.array_equal(g["meta"], O.store_meta(om)), "%s: metadata differs" % what
    oq, osw = O.quant_fp8(ov)
    assert f32_bits(g["sw"]) == f32_bits(osw), "%s: weight scale differs" % what
    assert np.array_equal(g["qv"], oq), "%s: %d weight codes differ" % (what, int((g["qv"] != oq).sum()))
    oxq, osx = O.quant_fp8(xb)
    assert f32_bits(g["sx"]) == f32_bits(osx), "%s: activation scale differs" % what
    assert np.array_equal(g["xq"], oxq), "%s: activation codes differ" % what
    del ov, wb
    w_hat = O.dequant_fp8(O.decompress(oq, om, k), osw)      # [n, k] float64
    w_abs = np.abs(w_hat)
    for m0 in range(0, m, block):
        x_hat = O.dequant_fp8(oxq[m0:m0 + block], osx)
        ref = x_hat @ w_hat.T
        mag = np.abs(x_hat) @ w_abs.T
        assert_within_tolerance(g["y"][m0:m0 + block], ref, mag, "%s tokens %d.." % (what, m0))


def test_prefill_full_size():
    _check(W.prefill_x(), W.prefill_weight(), "prefill")


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_layer_sweep_full_size(layer):
    for proj, (name, k, n) in enumerate(W.LAYER_PROJS):
        _check(W.layer_x(k), W.layer_weight(layer, proj), "layer %d %s" % (layer, name))
