"""GPU parity of the INT8 W8A8 path against the oracle: sp24_quant_int8 and
sp24_quant_int8_rows (bit-exact codes and scales), sp24_decompress on INT8
codes (bit-exact), and sp24_gemm / sp24_dense_gemm / sp24_gemm_rows with INT8
operands on every kernel the planner picks.

INT8 products are summed exactly in int32, so besides the library's general
tolerance the outputs meet a tight bound: the only rounding left is the int32
-> fp32 conversion, the fp32 scale product, split-K's fp32 sum of partials and
the bf16 output, so |y - ref| <= 2^-8 |ref| (1 + 2^-12) + 2^-20 mag."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (DEV, announce, assert_exact_sum_bound, assert_within_tolerance, bits, f32, f32_bits,
                         need_sp, u32)
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def i8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int8)


# ---------------------------------------------------------------- quantisers

@pytest.mark.parametrize("count", [1, 7, 4096, 131072, 131073, 1 << 20, 3 * (1 << 20) + 5])
def test_quant_int8_bit_exact(count):
    sp = need_sp()
    x = W.randn_bf16((count,), seed=count, std=3.0)
    announce("quant_int8", count)
    q, s = sp.quant_int8(x.to(DEV))
    torch.cuda.synchronize()
    oq, os_ = O.quant_int8(W.bf16_bits(x))
    assert f32_bits(f32(s)) == f32_bits(os_)
    got = i8(q)
    assert np.array_equal(got, oq), "codes differ in %d places" % int((got != oq).sum())
    assert got.min() >= -127


def test_quant_int8_static_ties_and_saturation():
    sp = need_sp()
    vals = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 127.5, 1000.0, -1000.0, 0.0] * 700,
                    dtype=np.float32)
    x = torch.from_numpy(vals).to(torch.bfloat16)
    announce("quant_int8 static", x.numel())
    scale = torch.ones(1, dtype=torch.float32, device=DEV)
    q, _ = sp.quant_int8(x.to(DEV), scale=scale)
    torch.cuda.synchronize()
    oq, _ = O.quant_int8(W.bf16_bits(x), scale=1.0)
    assert np.array_equal(i8(q), oq)
    assert i8(q)[:12].tolist() == [0, 2, 2, 0, -2, -2, 126, -126, 127, 127, -127, 0]


def test_quant_int8_zero_tensor():
    sp = need_sp()
    announce("quant_int8 zero")
    q, s = sp.quant_int8(torch.zeros(5000, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert f32(s) == 1.0 and not i8(q).any()


@pytest.mark.parametrize("m,k", [(1, 4096), (3, 136), (64, 14336), (257, 8192)])
def test_quant_int8_rows_bit_exact(m, k):
    sp = need_sp()
    x = W.randn_bf16((m, k), seed=m * 7 + k).float()
    if m > 2:
        x[m // 2] *= 1000.0
        x[m - 1] = 0.0
    x = x.to(torch.bfloat16)
    announce("quant_int8_rows", m, k)
    q, s = sp.quant_int8_rows(x.to(DEV))
    torch.cuda.synchronize()
    oq, os_ = O.quant_int8_rows(W.bf16_bits(x))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(i8(q), oq)


def test_decompress_int8_bit_exact():
    sp = need_sp()
    n, k = 96, 384
    w = W.randn_bf16((n, k), seed=3)
    announce("decompress int8", n, k)
    values, meta = sp.prune_compress(w.to(DEV))
    qv, _ = sp.quant_int8(values)
    wd = sp.decompress(qv, meta, k)
    torch.cuda.synchronize()
    ov, om = O.prune_compress(W.bf16_bits(w))
    oq, _ = O.quant_int8(ov)
    assert wd.dtype == torch.int8
    assert np.array_equal(i8(qv), oq)
    assert np.array_equal(i8(wd), O.decompress(oq, om, k))


# ---------------------------------------------------------------- GEMMs

# (m, n, k): stream (no split / split-K), skinny, tiled (ragged m and n)
SHAPES = [(1, 14336, 4096), (16, 14336, 4096), (64, 14336, 4096), (16, 1024, 16384), (3, 1000, 1024),
          (5, 300, 640), (1000, 8200, 640), (600, 32771, 384), (1111, 8198, 256)]


def _operands(m, n, k, seed):
    x = W.randn_bf16((m, k), seed=seed)
    w = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
    return x, w


def _oracle_weight(w):
    ov, om = O.prune_compress(W.bf16_bits(w))
    oq, osw = O.quant_int8(ov)
    return ov, om, oq, osw


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_int8_against_oracle(m, n, k):
    sp = need_sp()
    x, w = _operands(m, n, k, seed=m + 3 * n + k)
    pl = sp.plan(sp.OP_GEMM, sp.INT8, m, n, k)
    announce("gemm int8", m, n, k, "kernel", pl["kernel"], "split", pl["split_k"])
    values, meta = sp.prune_compress(w.to(DEV))
    qv, sw = sp.quant_int8(values)
    xq, sx = sp.quant_int8(x.to(DEV))
    y = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    _, om, oq, osw = _oracle_weight(w)
    oxq, osx = O.quant_int8(W.bf16_bits(x))
    assert np.array_equal(u32(meta), O.store_meta(om))
    assert f32_bits(f32(sw)) == f32_bits(osw) and f32_bits(f32(sx)) == f32_bits(osx)
    assert np.array_equal(i8(qv), oq) and np.array_equal(i8(xq), oxq)
    ref, mag = O.gemm_ref(*O.sparse_operands_int8(oxq, osx, oq, om, osw, k))
    yb = bits(y)
    assert_within_tolerance(yb, ref, mag, "gemm int8 %dx%dx%d" % (m, n, k))
    assert_exact_sum_bound(yb, ref, mag, "gemm int8 %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (16, 1024, 16384), (5, 300, 640), (1000, 8200, 640)])
def test_dense_gemm_int8_against_oracle(m, n, k):
    """The dense INT8 baseline multiplies the decompressed pruned weight."""
    sp = need_sp()
    x, w = _operands(m, n, k, seed=2 * m + n + k)
    announce("dense gemm int8", m, n, k, "kernel", sp.plan(sp.OP_DENSE_GEMM, sp.INT8, m, n, k)["kernel"])
    values, meta = sp.prune_compress(w.to(DEV))
    qv, sw = sp.quant_int8(values)
    wd = sp.decompress(qv, meta, k)
    xq, sx = sp.quant_int8(x.to(DEV))
    y = sp.dense_gemm(xq, wd, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    _, om, oq, osw = _oracle_weight(w)
    oxq, osx = O.quant_int8(W.bf16_bits(x))
    ref, mag = O.gemm_ref(*O.sparse_operands_int8(oxq, osx, oq, om, osw, k))
    yb = bits(y)
    assert_within_tolerance(yb, ref, mag, "dense int8 %dx%dx%d" % (m, n, k))
    assert_exact_sum_bound(yb, ref, mag, "dense int8 %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (16, 1024, 16384), (5, 300, 640), (600, 32771, 384)])
def test_gemm_rows_int8_against_oracle(m, n, k):
    sp = need_sp()
    x = W.randn_bf16((m, k), seed=5 * m + k).float()
    if m > 2:
        x[m // 2] *= 1000.0        # an outlier token
        x[m - 1] = 0.0             # an all-zero token
    x = x.to(torch.bfloat16)
    w = W.randn_bf16((n, k), seed=n + 9, std=0.02)
    announce("gemm_rows int8", m, n, k)
    values, meta = sp.prune_compress(w.to(DEV))
    qv, sw = sp.quant_int8(values)
    xq, xs = sp.quant_int8_rows(x.to(DEV))
    y = sp.gemm_rows(xq, qv, meta, xs, sw)
    torch.cuda.synchronize()
    _, om, oq, osw = _oracle_weight(w)
    oxq, oxs = O.quant_int8_rows(W.bf16_bits(x))
    ref, mag = O.gemm_ref(*O.sparse_operands_int8_rows(oxq, oxs, oq, om, osw, k))
    yb = bits(y)
    assert_within_tolerance(yb, ref, mag, "gemm_rows int8 %dx%dx%d" % (m, n, k))
    assert_exact_sum_bound(yb, ref, mag, "gemm_rows int8 %dx%dx%d" % (m, n, k))


def test_gemm_int8_extreme_codes_do_not_overflow():
    """Every code at +-127 along a long K: the largest sums the quantisers can make
    (127 * 127 * k/2, about 2^30 at k = 131072) stay exact in int32."""
    sp = need_sp()
    m, n, k = 2, 64, 131072
    announce("gemm int8 extreme", m, n, k)
    x = torch.full((m, k), 127, dtype=torch.int8, device=DEV)
    x[1] = -127
    wb = torch.full((n, k), 127.0, dtype=torch.bfloat16, device=DEV)
    wb[:, 1::4] = 0.0               # each group of 4 keeps positions 0 and 3
    wb[:, 2::4] = 0.0
    values, meta = sp.prune_compress(wb)
    qv = values.to(torch.float32).to(torch.int8).contiguous()
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    y = sp.gemm(x, qv, meta, x_scale=one, w_scale=one)
    torch.cuda.synchronize()
    expect = torch.tensor([127.0 * 127.0 * (k // 2)], dtype=torch.float32).to(torch.bfloat16).float().item()
    yf = y.float().cpu()
    assert bool((yf[0] == expect).all()) and bool((yf[1] == -expect).all())


def test_gemm_int8_repeatable():
    sp = need_sp()
    m, n, k = 64, 14336, 4096
    x, w = _operands(m, n, k, seed=77)
    announce("gemm int8 repeat", m, n, k)
    values, meta = sp.prune_compress(w.to(DEV))
    qv, sw = sp.quant_int8(values)
    xq, sx = sp.quant_int8(x.to(DEV))
    y1 = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    y2 = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def _sampled_int8(x_cpu, w_cpu, what, n_rows=256, n_tokens=None, seed=0):
    """Full-size INT8 run of the bench shapes; the oracle checks sampled W rows and tokens
    (scales from every value: the per-tensor maximum survives 2:4 pruning)."""
    sp = need_sp()
    announce("gemm int8 sampled", what, tuple(x_cpu.shape), tuple(w_cpu.shape))
    values, meta = sp.prune_compress(w_cpu.to(DEV))
    qv, sw = sp.quant_int8(values)
    xq, sx = sp.quant_int8(x_cpu.to(DEV))
    y = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    n, m, k = w_cpu.shape[0], x_cpu.shape[0], w_cpu.shape[1]
    rows = np.unique(np.concatenate([np.sort(rng.choice(n, size=min(n_rows, n), replace=False)), [0, n - 1]]))
    toks = np.arange(m) if n_tokens is None else np.unique(np.concatenate(
        [np.sort(rng.choice(m, size=n_tokens, replace=False)), [0, m - 1]]))
    wb, xb = W.bf16_bits(w_cpu), W.bf16_bits(x_cpu)
    ov, om = O.prune_compress(wb[rows])
    osw = O.int8_scale(wb)
    oq, _ = O.quant_int8(ov, scale=osw)
    osx = O.int8_scale(xb)
    oxq, _ = O.quant_int8(xb[toks], scale=osx)
    assert f32_bits(f32(sw)) == f32_bits(osw) and f32_bits(f32(sx)) == f32_bits(osx)
    assert np.array_equal(i8(qv)[rows], oq)
    assert np.array_equal(i8(xq)[toks], oxq)
    assert np.array_equal(O.load_meta(u32(meta), n, k, rows), om)
    ref, mag = O.gemm_ref(*O.sparse_operands_int8(oxq, osx, oq, om, osw, k))
    yb = bits(y)[np.ix_(toks, rows)]
    assert_within_tolerance(yb, ref, mag, what)
    assert_exact_sum_bound(yb, ref, mag, what)


def test_prefill_sampled_int8():
    _sampled_int8(W.prefill_x(), W.prefill_weight(), "prefill int8", n_rows=256, n_tokens=256)


@pytest.mark.parametrize("m", [1, 16, 64])
def test_decode_sampled_int8(m):
    _sampled_int8(W.up_x(m), W.up_weight(), "up int8 M=%d" % m, seed=m)
    _sampled_int8(W.down_x(m), W.down_weight(), "down int8 M=%d" % m, seed=m + 1)


@pytest.mark.parametrize("m,n,k,sk", [(256, 1000, 1024, 2), (300, 520, 2048, 4)])
def test_gemm_int8_tiled_split_k(m, n, k, sk):
    """INT8 through the tiled kernel with its K split: per-slice int32 sums become fp32
    partials, summed by the reduction in a fixed order."""
    import os
    os.environ["SP24_TILE"] = "99,%d" % sk
    try:
        test_gemm_int8_against_oracle(m, n, k)
    finally:
        os.environ.pop("SP24_TILE", None)
