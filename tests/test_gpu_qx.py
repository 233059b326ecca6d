"""GPU parity of sp24_gemm_qx (X quantised inside the GEMM at decode sizes).

The call must equal sp24_quant_fp8 (dynamic per-tensor scale) followed by
sp24_gemm bit for bit, in Y and in the stored scale, whether X is quantised
inside the stream kernel or by the two-launch path; and Y must meet the
oracle's tolerance like every GEMM.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import sp24_ref as O
from gpu_helpers import (DEV, GpuWeight, OracleWeight, announce, assert_within_tolerance, bits, f32,
                         f32_bits, need_sp, oracle_ref, oracle_x)

pytestmark = pytest.mark.gpu

# (m, n, k, quantised inside the kernel)
SHAPES = [(1, 14336, 4096, True), (1, 4096, 14336, True),
          (3, 1000, 1024, True),        # split-K over 2 slices, ragged rows
          (1, 1024, 16384, True),       # split-K over 4 slices
          (16, 40, 4096, True),         # split-K over 8 slices, 3 workgroups of rows
          (40, 4096, 512, True),        # two token groups of 32 rows (the second ragged)
          (2, 512, 16384, True),        # split-K over 8 slices, two tokens; X read twice (4 waves)
          (4, 14336, 4096, True),       # 4 tokens over all of K, X in registers
          (16, 14336, 4096, False),     # 16 tokens over all of K: too many values to cast per workgroup
          (4, 4096, 14336, False),
          (5, 300, 640, False),         # small-m kernel without LDS: two launches
          (64, 14336, 4096, False),     # X too large to quantise in every workgroup
          (16, 4096, 14336, False)]


def _fused(sp, m, n, k):
    g = sp.lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)
    return sp.lib.sp24_workspace_size(sp.OP_GEMM_QX, sp.FP8, m, n, k) == (g + 15) // 16 * 16


@pytest.mark.parametrize("m,n,k,fused", SHAPES)
def test_gemm_qx_equals_quant_then_gemm(m, n, k, fused):
    sp = need_sp()
    assert _fused(sp, m, n, k) == fused
    seed = 7 * m + 3 * n + k
    x_cpu = W.randn_bf16((m, k), seed=seed)
    w_cpu = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
    announce("gemm_qx", m, n, k, "fused" if fused else "two launches")
    gw = GpuWeight(w_cpu, True)
    x = x_cpu.to(DEV)
    y, sx = sp.gemm_qx(x, gw.qvalues, gw.meta, gw.scale)
    xq2, sx2 = sp.quant_fp8(x)
    y2 = sp.gemm(xq2, gw.qvalues, gw.meta, x_scale=sx2, w_scale=gw.scale)
    torch.cuda.synchronize()
    assert f32_bits(f32(sx)) == f32_bits(f32(sx2))
    assert np.array_equal(bits(y), bits(y2)), "differs from quantise + GEMM in %d outputs" % int(
        (bits(y) != bits(y2)).sum())
    ow = OracleWeight(W.bf16_bits(w_cpu), True)
    oxq, oxs = oracle_x(W.bf16_bits(x_cpu), True)
    assert f32_bits(f32(sx)) == f32_bits(oxs)
    ref, mag = oracle_ref(oxq, oxs, ow)
    assert_within_tolerance(bits(y), ref, mag, "gemm_qx %dx%dx%d" % (m, n, k))


def test_gemm_qx_scale_from_the_last_value_and_zero_input():
    """The per-tensor maximum can sit anywhere in X; every workgroup must see it."""
    sp = need_sp()
    m, n, k = 3, 1000, 1024
    w_cpu = W.randn_bf16((n, k), seed=5, std=0.02)
    gw = GpuWeight(w_cpu, True)
    x_cpu = W.randn_bf16((m, k), seed=6)
    x_cpu[m - 1, k - 1] = -300.0                     # the largest magnitude, last element
    announce("gemm_qx amax at the end")
    y, sx = sp.gemm_qx(x_cpu.to(DEV), gw.qvalues, gw.meta, gw.scale)
    torch.cuda.synchronize()
    oxq, oxs = oracle_x(W.bf16_bits(x_cpu), True)
    assert f32_bits(f32(sx)) == f32_bits(oxs)
    ref, mag = oracle_ref(oxq, oxs, OracleWeight(W.bf16_bits(w_cpu), True))
    assert_within_tolerance(bits(y), ref, mag, "gemm_qx amax at the end")
    announce("gemm_qx zero input")
    y0, s0 = sp.gemm_qx(torch.zeros(m, k, dtype=torch.bfloat16, device=DEV), gw.qvalues, gw.meta, gw.scale)
    torch.cuda.synchronize()
    assert float(f32(s0)) == 1.0
    assert not bits(y0).any() or np.all((bits(y0) & 0x7FFF) == 0)


def test_gemm_qx_repeated_calls_are_bitwise_stable():
    sp = need_sp()
    m, n, k = 16, 14336, 4096
    gw = GpuWeight(W.up_weight(), True)
    x = W.up_x(m).to(DEV)
    announce("gemm_qx repeated")
    ys = [bits(sp.gemm_qx(x, gw.qvalues, gw.meta, gw.scale)[0]) for _ in range(3)]
    assert all(np.array_equal(ys[0], yy) for yy in ys[1:])


# ---------------------------------------------------------------- one scale per token

def _fused_rows(sp, m, n, k):
    g = sp.lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)
    return sp.lib.sp24_workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, n, k) == (g + 15) // 16 * 16


@pytest.mark.parametrize("m,n,k,fused", SHAPES)
def test_gemm_rows_qx_equals_quant_rows_then_gemm_rows(m, n, k, fused):
    """sp24_gemm_rows_qx = sp24_quant_fp8_rows + sp24_gemm_rows bit for bit (Y and every row's
    scale), fused into the stream kernel or not, and within the oracle's tolerance."""
    sp = need_sp()
    assert _fused_rows(sp, m, n, k) == fused
    seed = 5 * m + 3 * n + k
    x_cpu = W.randn_bf16((m, k), seed=seed).float()
    if m > 2:
        x_cpu[m // 2] *= 300.0        # an outlier token
        x_cpu[m - 1] = 0.0            # an all-zero token: scale 1
    x_cpu = x_cpu.to(torch.bfloat16)
    w_cpu = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
    announce("gemm_rows_qx", m, n, k, "fused" if fused else "two launches")
    gw = GpuWeight(w_cpu, True)
    x = x_cpu.to(DEV)
    y, sx = sp.gemm_rows_qx(x, gw.qvalues, gw.meta, gw.scale)
    xq2, sx2 = sp.quant_fp8_rows(x)
    y2 = sp.gemm_rows(xq2, gw.qvalues, gw.meta, sx2, gw.scale)
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx2.cpu().numpy().view(np.uint32))
    assert np.array_equal(bits(y), bits(y2)), "differs from quant_rows + gemm_rows in %d outputs" % int(
        (bits(y) != bits(y2)).sum())
    ow = OracleWeight(W.bf16_bits(w_cpu), True)
    oxq, oxs = O.quant_fp8_rows(W.bf16_bits(x_cpu))
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), oxs.view(np.uint32))
    ref, mag = O.gemm_ref(*O.sparse_operands_fp8_rows(oxq, oxs, ow.qvalues, ow.meta, ow.scale, k))
    assert_within_tolerance(bits(y), ref, mag, "gemm_rows_qx %dx%dx%d" % (m, n, k))


def test_gemm_rows_qx_repeated_calls_are_bitwise_stable():
    sp = need_sp()
    gw = GpuWeight(W.up_weight(), True)
    for m in (1, 2):
        x = W.up_x(m).to(DEV)
        announce("gemm_rows_qx repeated", m)
        ys = [bits(sp.gemm_rows_qx(x, gw.qvalues, gw.meta, gw.scale)[0]) for _ in range(3)]
        assert all(np.array_equal(ys[0], yy) for yy in ys[1:])
