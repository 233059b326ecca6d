"""GPU parity of the per-token path: sp24_quant_fp8_rows (bit-exact codes and
scales) and sp24_gemm_rows (oracle tolerance) on every kernel the planner picks."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (DEV, GpuWeight, OracleWeight, announce, assert_within_tolerance, bits, codes,
                         need_sp)
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _x_with_outliers(m, k, seed):
    x = W.randn_bf16((m, k), seed=seed).float()
    if m > 2:
        x[m // 2] *= 1000.0        # an outlier token
        x[m - 1] = 0.0             # an all-zero token
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("m,k", [(1, 4096), (3, 136), (64, 14336), (257, 8192), (5, 8200)])
def test_quant_rows_bit_exact(m, k):
    sp = need_sp()
    x = _x_with_outliers(m, k, seed=m * 31 + k)
    announce("quant_fp8_rows", m, k)
    q, s = sp.quant_fp8_rows(x.to(DEV))
    torch.cuda.synchronize()
    oq, os_ = O.quant_fp8_rows(W.bf16_bits(x))
    gs = s.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"
    assert np.array_equal(codes(q), oq), "codes differ in %d places" % int((codes(q) != oq).sum())


# (m, n, k): stream (no split / split-K), skinny, tiled (ragged m and n)
GEMM_SHAPES = [(1, 14336, 4096), (16, 14336, 4096), (64, 14336, 4096), (16, 1024, 16384), (3, 1000, 1024),
               (5, 300, 640), (1000, 8200, 640), (600, 32771, 384)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_rows_against_oracle(m, n, k):
    sp = need_sp()
    x = _x_with_outliers(m, k, seed=m + n + k)
    w = W.randn_bf16((n, k), seed=m + n + k + 1, std=0.02)
    announce("gemm_rows", m, n, k, "kernel", sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)["kernel"])
    gw = GpuWeight(w, True)
    xq, xs = sp.quant_fp8_rows(x.to(DEV))
    y = sp.gemm_rows(xq, gw.qvalues, gw.meta, xs, gw.scale)
    torch.cuda.synchronize()
    ow = OracleWeight(W.bf16_bits(w), True)
    oxq, oxs = O.quant_fp8_rows(W.bf16_bits(x))
    ref, mag = O.gemm_ref(*O.sparse_operands_fp8_rows(oxq, oxs, ow.qvalues, ow.meta, ow.scale, k))
    assert_within_tolerance(bits(y), ref, mag, "gemm_rows %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(16, 14336, 4096), (16, 1024, 16384), (1000, 8200, 640), (5, 300, 640)])
def test_gemm_rows_with_equal_scales_is_gemm(m, n, k):
    """With every row scale equal to the tensor's scale the two epilogues are the same product."""
    sp = need_sp()
    x = W.randn_bf16((m, k), seed=11 * m + k).to(DEV)
    gw = GpuWeight(W.randn_bf16((n, k), seed=n + 5, std=0.02), True)
    announce("gemm_rows equal scales", m, n, k)
    xq, sx = sp.quant_fp8(x)
    y1 = sp.gemm(xq, gw.qvalues, gw.meta, x_scale=sx, w_scale=gw.scale)
    y2 = sp.gemm_rows(xq, gw.qvalues, gw.meta, sx.expand(m).contiguous(), gw.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
