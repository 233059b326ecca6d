"""GPU parity of the SlideSparse path ("SlideSparse: Fast and Flexible
(2N-2):2N Structured Sparsity"): the packed weight and the lifted codes are
bit-exact with the oracle, and the 2:4 GEMM over K' gives the (2N-2):2N
product over K within the GEMM tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (DEV, announce, assert_exact_sum_bound, assert_within_tolerance, bits, codes, f32, f32_bits,
                         need_sp, u32)
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _oracle_pack(wb, n_pat):
    return O.slide_pack(O.apply_mask(wb, O.slide_prune_mask(wb, n_pat)), n_pat)


@pytest.mark.parametrize("n,k,n_pat", [(5, 64, 4), (33, 4096, 4), (7, 96, 3), (9, 160, 5), (4, 256, 8)])
def test_prune_pack_bit_exact(n, k, n_pat):
    sp = need_sp()
    rng = np.random.default_rng(n * k + n_pat)
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0], dtype=np.float32)
    for what, w in (("normal", W.randn_bf16((n, k), seed=n + k, std=0.02)),
                    ("ties", torch.from_numpy(rng.choice(alphabet, size=(n, k))).to(torch.bfloat16))):
        announce("slide_prune_pack", what, n, k, n_pat)
        wp = sp.slide_prune_pack(w.to(DEV), n_pat)
        torch.cuda.synchronize()
        ref = _oracle_pack(W.bf16_bits(w), n_pat)
        got = bits(wp)
        assert np.array_equal(got, ref), "%s: %d values differ" % (what, int((got != ref).sum()))


@pytest.mark.parametrize("m,k,n_pat", [(1, 4096, 4), (16, 14336, 4), (5, 96, 3), (3, 160, 5)])
def test_lift_quant_bit_exact(m, k, n_pat):
    sp = need_sp()
    x = W.randn_bf16((m, k), seed=m + k).float()
    if m > 2:
        x[1] *= 300.0
    x = x.to(torch.bfloat16)
    announce("slide_quant_fp8_rows", m, k, n_pat)
    q, s = sp.slide_quant_fp8_rows(x.to(DEV), n_pat)
    torch.cuda.synchronize()
    oq, os_ = O.quant_fp8_rows(W.bf16_bits(x))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(codes(q), O.slide_lift(oq, n_pat))


# (m, n, k): stream without and with split-K, tiled
@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (16, 1024, 4096), (64, 2048, 2048), (512, 16384, 1024)])
def test_slide_gemm_matches_the_6_of_8_product(m, n, k):
    sp = need_sp()
    n_pat = 4
    w = W.randn_bf16((n, k), seed=n + k, std=0.02)
    x = W.randn_bf16((m, k), seed=m + k + 1)
    kp = k * (2 * n_pat - 2) // n_pat
    announce("slide gemm", m, n, k, "K'", kp, "kernel", sp.plan(sp.OP_GEMM, sp.FP8, m, n, kp)["kernel"])
    wp = sp.slide_prune_pack(w.to(DEV), n_pat)
    values, meta = sp.prune_compress(wp)
    qv, sw = sp.quant_fp8(values)
    xq, sx = sp.slide_quant_fp8_rows(x.to(DEV), n_pat)
    y = sp.gemm_rows(xq, qv, meta, sx, sw)
    torch.cuda.synchronize()
    # the weight: 6:8 pruned, per-tensor scale (W' holds exactly its nonzero values)
    wb = W.bf16_bits(w)
    w68 = O.apply_mask(wb, O.slide_prune_mask(wb, n_pat))
    wq, osw = O.quant_fp8(w68)
    assert f32_bits(f32(sw)) == f32_bits(osw)
    ov, om = O.prune_compress(O.slide_pack(w68, n_pat))
    assert np.array_equal(u32(meta), O.store_meta(om))      # the 2:4 prune kept every value
    oxq, oxs = O.quant_fp8_rows(W.bf16_bits(x))
    ref, mag = O.gemm_ref(O.dequant_fp8_rows(oxq, oxs), O.dequant_fp8(wq, osw))
    assert_within_tolerance(bits(y), ref, mag, "slide %dx%dx%d" % (m, n, k))


# ---------------------------------------------------------------- INT8 W8A8 (the page's precision)

@pytest.mark.parametrize("m,k,n_pat", [(1, 4096, 4), (16, 14336, 4), (5, 96, 3), (3, 160, 5), (2, 256, 8)])
def test_lift_quant_int8_bit_exact(m, k, n_pat):
    sp = need_sp()
    x = W.randn_bf16((m, k), seed=3 * m + k).float()
    if m > 2:
        x[1] *= 300.0
        x[2] = 0.0                 # an all-zero token: scale 1, codes 0
    x = x.to(torch.bfloat16)
    announce("slide_quant_int8_rows", m, k, n_pat)
    q, s = sp.slide_quant_int8_rows(x.to(DEV), n_pat)
    torch.cuda.synchronize()
    oq, os_ = O.quant_int8_rows(W.bf16_bits(x))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), O.slide_lift(oq, n_pat))


@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (16, 1024, 4096), (64, 2048, 2048), (512, 16384, 1024)])
def test_slide_gemm_int8_matches_the_6_of_8_product(m, n, k):
    sp = need_sp()
    n_pat = 4
    w = W.randn_bf16((n, k), seed=n + k + 2, std=0.02)
    x = W.randn_bf16((m, k), seed=m + k + 3)
    kp = k * (2 * n_pat - 2) // n_pat
    announce("slide gemm int8", m, n, k, "K'", kp, "kernel", sp.plan(sp.OP_GEMM, sp.INT8, m, n, kp)["kernel"])
    wp = sp.slide_prune_pack(w.to(DEV), n_pat)
    values, meta = sp.prune_compress(wp)
    qv, sw = sp.quant_int8(values)
    xq, sx = sp.slide_quant_int8_rows(x.to(DEV), n_pat)
    y = sp.gemm_rows(xq, qv, meta, sx, sw)
    torch.cuda.synchronize()
    # the reference over K: 6:8-pruned W with its per-tensor INT8 scale, X per token
    wb = W.bf16_bits(w)
    w68 = O.apply_mask(wb, O.slide_prune_mask(wb, n_pat))
    wq, osw = O.quant_int8(w68)
    assert f32_bits(f32(sw)) == f32_bits(osw)
    oxq, oxs = O.quant_int8_rows(W.bf16_bits(x))
    xs = oxs.astype(np.float64)[:, None] * oxq.astype(np.float64)
    ref, mag = O.gemm_ref(xs, O.dequant_int8(wq, osw))
    yb = bits(y)
    assert_within_tolerance(yb, ref, mag, "slide int8 %dx%dx%d" % (m, n, k))
    assert_exact_sum_bound(yb, ref, mag, "slide int8 %dx%dx%d" % (m, n, k))


# ---------------------------------------------------------------- lifting fused into the GEMM

# (m, n, k, N, lifted inside the GEMM kernel): no split, split-K over 2/4/8 slices (slice
# boundaries inside the lifted blocks), ragged rows, and shapes that take two launches
SLIDE_QX = [(1, 14336, 4096, 4, True), (2, 14336, 4096, 4, True), (1, 1024, 6144, 3, True),
            (3, 1000, 5120, 5, True), (1, 1024, 4096, 8, True), (2, 512, 16384, 4, True),
            (1, 40, 8192, 4, True), (4, 300, 2560, 5, True),
            (16, 1024, 4096, 4, False), (3, 1000, 1536, 4, False), (1, 4096, 14336, 4, False),
            (64, 2048, 4096, 4, False)]


@pytest.mark.parametrize("m,n,k,n_pat,fused", SLIDE_QX)
def test_slide_gemm_qx_equals_lift_quant_then_gemm_rows(m, n, k, n_pat, fused):
    """sp24_slide_gemm_qx = sp24_slide_quant_fp8_rows + sp24_gemm_rows over K' bit for bit (Y
    and every row's scale), and within the oracle's tolerance of the (2N-2):2N product."""
    sp = need_sp()
    kp = k // (2 * n_pat) * 4 * (n_pat - 1)
    g = sp.lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, kp)
    assert (sp.lib.sp24_workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, n, kp) == (g + 15) // 16 * 16) == fused
    w = W.randn_bf16((n, k), seed=n + k + n_pat, std=0.02)
    x = W.randn_bf16((m, k), seed=m + k + 5).float()
    if m > 2:
        x[1] *= 300.0
        x[m - 1] = 0.0
    x = x.to(torch.bfloat16)
    announce("slide_gemm_qx", m, n, k, "N", n_pat, "K'", kp, "fused" if fused else "two launches")
    wp = sp.slide_prune_pack(w.to(DEV), n_pat)
    values, meta = sp.prune_compress(wp)
    qv, sw = sp.quant_fp8(values)
    y, sx = sp.slide_gemm_qx(x.to(DEV), qv, meta, sw, n_pat)
    xq2, sx2 = sp.slide_quant_fp8_rows(x.to(DEV), n_pat)
    y2 = sp.gemm_rows(xq2, qv, meta, sx2, sw)
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx2.cpu().numpy().view(np.uint32))
    assert np.array_equal(bits(y), bits(y2)), "differs from lift + quant + gemm_rows in %d outputs" % int(
        (bits(y) != bits(y2)).sum())
    # the reference over K: the (2N-2):2N-pruned W, per-tensor W scale, per-token X scales
    wb = W.bf16_bits(w)
    wpr = O.apply_mask(wb, O.slide_prune_mask(wb, n_pat))
    wq, osw = O.quant_fp8(wpr)
    oxq, oxs = O.quant_fp8_rows(W.bf16_bits(x))
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), oxs.view(np.uint32))
    ref, mag = O.gemm_ref(O.dequant_fp8_rows(oxq, oxs), O.dequant_fp8(wq, osw))
    assert_within_tolerance(bits(y), ref, mag, "slide_gemm_qx %dx%dx%d N=%d" % (m, n, k, n_pat))
