"""GPU parity at sizes past 2^31 elements (64-bit indexing in every kernel).

Inputs are drawn on the GPU from seeded generators (drawing 2^31 values on the
host would take minutes); the oracle checks sampled rows and tokens, and every
whole-tensor property it can take (the per-tensor scales) from all values.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, OracleWeight, announce, assert_within_tolerance, bits, codes, f32,
                         f32_bits, need_sp, oracle_ref, u32)
from oracle import sp24_ref as O

pytestmark = pytest.mark.gpu


def _gpu_randn_bf16(shape, seed, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    rows = max(1, (1 << 26) // shape[-1])  # draw in pieces of ~64 M floats
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        out[r0:r1] = (torch.randn(r1 - r0, shape[-1], generator=g, device=DEV) * std).to(torch.bfloat16)
    return out


def test_weight_past_2_31_elements_prune_quant_gemm():
    sp = need_sp()
    n, k = 65536, 32768                      # 2^31 weight elements, 4 GiB of bf16
    announce("large weight", n, k)
    w = _gpu_randn_bf16((n, k), seed=91, std=0.02)
    values, meta = sp.prune_compress(w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(n, size=192, replace=False), [0, n - 1]]))
    wb = bits(w[torch.from_numpy(rows).to(DEV)])
    del w
    ov, om = O.prune_compress(wb)
    assert np.array_equal(bits(values)[rows], ov)
    assert np.array_equal(O.load_meta(u32(meta), n, k, rows), om)

    qv, sw = sp.quant_fp8(values)            # 2^30 values: the two-launch quantiser
    torch.cuda.synchronize()
    s_ref = O.fp8_scale(bits(values).reshape(-1))
    assert f32_bits(f32(sw)) == f32_bits(s_ref)
    q_ref, _ = O.quant_fp8(ov, scale=s_ref)
    assert np.array_equal(codes(qv)[rows], q_ref)

    for m in (1, 16):
        x = _gpu_randn_bf16((m, k), seed=92 + m)
        xq, sx = sp.quant_fp8(x)
        y = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
        torch.cuda.synchronize()
        oxs = O.fp8_scale(bits(x))
        oxq, _ = O.quant_fp8(bits(x), scale=oxs)
        assert f32_bits(f32(sx)) == f32_bits(oxs)
        assert np.array_equal(codes(xq), oxq)
        ow = SimpleNamespace(fp8=True, k=k, values=ov, meta=om, qvalues=q_ref, scale=s_ref)
        ref, mag = oracle_ref(oxq, oxs, ow)
        assert_within_tolerance(bits(y)[:, rows], ref, mag, "large weight M=%d" % m)


def test_activation_past_2_31_values_quant_and_prefill_gemm():
    sp = need_sp()
    m, n, k = 65536, 512, 32768              # X has 2^31 values
    announce("large activation", m, n, k)
    x = _gpu_randn_bf16((m, k), seed=93)
    xq, sx = sp.quant_fp8(x)
    torch.cuda.synchronize()
    oxs = O.fp8_scale(bits(x).reshape(-1))
    assert f32_bits(f32(sx)) == f32_bits(oxs)
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([rng.choice(m, size=96, replace=False), [0, m - 1]]))
    xb = bits(x[torch.from_numpy(toks).to(DEV)])
    del x
    oxq, _ = O.quant_fp8(xb, scale=oxs)
    assert np.array_equal(codes(xq)[toks], oxq)

    w = _gpu_randn_bf16((n, k), seed=94, std=0.02)
    values, meta = sp.prune_compress(w)
    qv, sw = sp.quant_fp8(values)
    assert sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)["kernel"] == 1   # the LDS-tiled kernel
    y = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
    torch.cuda.synchronize()
    ow = OracleWeight(bits(w), True)
    assert f32_bits(f32(sw)) == f32_bits(ow.scale)
    assert np.array_equal(codes(qv), ow.qvalues)
    ref, mag = oracle_ref(oxq, oxs, ow)
    assert_within_tolerance(bits(y)[toks], ref, mag, "large activation")
