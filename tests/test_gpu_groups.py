"""GPU parity of the finer FP8 scales: sp24_quant_fp8_groups (codes and scales bit-exact
against the oracle) and sp24_gemm_groups (oracle tolerance) for 128-K groups, wider groups
and one group per row (per-token X, per-output-channel W), on every kernel the planner
picks: the stream kernel with its table of group scales (with and without split-K, and at
large m), and for one group per row the stream, skinny and tiled kernels."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, announce, assert_within_tolerance, bits, codes, need_sp
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _x(m, k, seed):
    x = W.randn_bf16((m, k), seed=seed).float()
    x[:, (seed % 7)::97] *= 30.0      # outlier channels: one group's scale differs from its neighbours'
    if m > 2:
        x[m - 1] = 0.0                # an all-zero token: scales 1, codes 0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols,group", [(1, 4096, 128), (64, 14336, 128), (5, 384, 8), (7, 1152, 384),
                                             (14336, 2048, 64), (300, 2048, 2048), (3, 7168, 7168),
                                             (2, 200, 40)])
def test_quant_groups_bit_exact(rows, cols, group):
    sp = need_sp()
    x = _x(rows, cols, seed=rows * 3 + cols + group)
    announce("quant_fp8_groups", rows, cols, group)
    q, s = sp.quant_fp8_groups(x.to(DEV), group)
    torch.cuda.synchronize()
    oq, os_ = O.quant_fp8_groups(W.bf16_bits(x), group)
    assert np.array_equal(s.cpu().numpy().reshape(os_.shape).view(np.uint32), os_.view(np.uint32)), "scales differ"
    assert np.array_equal(codes(q), oq), "codes differ in %d places" % int((codes(q) != oq).sum())


class _Case:
    """Both sides of one grouped product: the HIP path through the binding (weight pruned,
    compressed and quantised in groups of group/2 kept values; X quantised in groups) and
    the oracle's float64 reference on the oracle's own codes and scales."""

    def __init__(self, m, n, k, group, seed):
        sp = need_sp()
        x = _x(m, k, seed)
        w = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
        values, meta = sp.prune_compress(w.to(DEV))
        self.wq, self.ws = sp.quant_fp8_groups(values, group // 2)
        self.meta = meta
        self.xq, self.xs = sp.quant_fp8_groups(x.to(DEV), group)
        ov, om = O.prune_compress(W.bf16_bits(w))
        owq, ows = O.quant_fp8_groups(ov, group // 2)
        oxq, oxs = O.quant_fp8_groups(W.bf16_bits(x), group)
        torch.cuda.synchronize()
        assert np.array_equal(codes(self.wq), owq) and np.array_equal(codes(self.xq), oxq)
        assert np.array_equal(self.ws.cpu().numpy().reshape(ows.shape), ows)
        assert np.array_equal(self.xs.cpu().numpy().reshape(oxs.shape), oxs)
        self.ref, self.mag = O.gemm_ref(*O.sparse_operands_fp8_groups(oxq, oxs, owq, om, ows, k, group))
        self.group = group

    def run(self):
        sp = need_sp()
        y = sp.gemm_groups(self.xq, self.xs, self.wq, self.meta, self.ws, self.group)
        torch.cuda.synchronize()
        return bits(y)


# (m, n, k, group): decode up and down (the down-projection splits K), ragged shapes,
# groups wider than 128, one group per row on the stream, skinny and tiled kernels
SHAPES = [(1, 14336, 4096, 128), (16, 14336, 4096, 128), (64, 14336, 4096, 128),
          (1, 4096, 14336, 128), (16, 4096, 14336, 128), (64, 4096, 14336, 128),
          (37, 1000, 1152, 128), (3, 300, 640, 128), (300, 520, 1024, 128),
          (64, 4096, 14336, 512), (16, 2048, 3584, 896), (5, 1000, 2048, 256),
          (64, 14336, 4096, 4096), (1, 4096, 14336, 14336), (5, 300, 640, 640), (600, 1000, 768, 768),
          (3, 1000, 1152, 1152)]


@pytest.mark.parametrize("m,n,k,group", SHAPES)
def test_gemm_groups_against_oracle(m, n, k, group):
    sp = need_sp()
    plan = sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)
    announce("gemm_groups", m, n, k, group, "plan kernel", plan["kernel"], "config", plan["config"])
    c = _Case(m, n, k, group, seed=m + n + k + group)
    assert_within_tolerance(c.run(), c.ref, c.mag, "gemm_groups %dx%dx%d/%d" % (m, n, k, group))


def test_gemm_groups_is_bitwise_reproducible():
    c = _Case(64, 4096, 14336, 128, seed=5)
    announce("gemm_groups repeat")
    a, b = c.run(), c.run()
    assert np.array_equal(a, b)


def test_one_group_with_equal_scales_is_the_per_tensor_gemm():
    """group == k with every X row scale equal and every W channel scale equal is sp24_gemm
    with per-tensor scales, bit for bit (the same kernels, the same epilogue products)."""
    sp = need_sp()
    m, n, k = 16, 14336, 4096
    x = W.randn_bf16((m, k), seed=3).to(DEV)
    w = W.randn_bf16((n, k), seed=4, std=0.02).to(DEV)
    announce("gemm_groups equal scales", m, n, k)
    values, meta = sp.prune_compress(w)
    wq, sw = sp.quant_fp8(values)
    xq, sx = sp.quant_fp8(x)
    y1 = sp.gemm(xq, wq, meta, x_scale=sx, w_scale=sw)
    y2 = sp.gemm_groups(xq, sx.expand(m).contiguous(), wq, meta, sw.expand(n).contiguous(), k)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))


def test_prefill_groups_sampled():
    """Prefill-sized products, rows and tokens sampled: one group per row on the tiled
    kernel (2048 tokens x 4096 rows), and 128-K groups (on the stream kernel)."""
    sp = need_sp()
    m, n, k = 2048, 4096, 4096
    x = _x(m, k, seed=77)
    w = W.randn_bf16((n, k), seed=78, std=0.01)
    values, meta = sp.prune_compress(w.to(DEV))
    ov, om = O.prune_compress(W.bf16_bits(w))
    rows = np.r_[0:64, n - 64:n]
    toks = np.r_[0:96, m - 32:m]
    for group in (k, 128):
        announce("gemm_groups prefill", m, n, k, group)
        wq, ws = sp.quant_fp8_groups(values, group // 2)
        xq, xs = sp.quant_fp8_groups(x.to(DEV), group)
        y = sp.gemm_groups(xq, xs, wq, meta, ws, group)
        torch.cuda.synchronize()
        owq, ows = O.quant_fp8_groups(ov[rows], group // 2)
        oxq, oxs = O.quant_fp8_groups(W.bf16_bits(x)[toks], group)
        ometa = om[rows]
        ref, mag = O.gemm_ref(*O.sparse_operands_fp8_groups(oxq, oxs, owq, ometa, ows, k, group))
        assert_within_tolerance(bits(y)[np.ix_(toks, rows)], ref, mag, "prefill groups %d" % group)
