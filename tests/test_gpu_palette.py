"""GPU parity of the exponent-palette path against the oracle: the encoding
(palette, row lists, sign+mantissa bytes, index words, verbatim rows) and the
lossless decode bit for bit, and sp24_palette_gemm on both pipelines (m <= 16:
BF16 rebuilt in registers; m > 16: rebuilt W + dense GEMM) within the GEMM
tolerance of the float64 product of the original weight."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, announce, assert_within_tolerance, bits, need_sp
from oracle import palette_ref as P

pytestmark = pytest.mark.gpu


def _weights(kind, n, k, seed):
    if kind == "gauss":
        return W.randn_bf16((n, k), seed=seed, std=0.02)
    if kind == "few":          # 4 exponents: no verbatim row
        g = torch.Generator().manual_seed(seed)
        return (torch.randint(1, 16, (n, k), generator=g).float() / 4.0 *
                torch.where(torch.rand(n, k, generator=g) < 0.5, -1.0, 1.0)).to(torch.bfloat16)
    if kind == "allverb":      # 16 common exponents in every row plus a rare one in every row
        base = torch.tensor(2.0 ** (np.arange(k) % 16), dtype=torch.float32).repeat(n, 1)
        for r in range(n):
            base[r, (7 * r) % k] = 2.0 ** (-60 - (r % 40))
        return base.to(torch.bfloat16)
    raise ValueError(kind)


def _encode_and_check(w):
    sp = need_sp()
    pw = sp.palette_encode(w.to(DEV))
    torch.cuda.synchronize()
    enc = P.palette_encode(W.bf16_bits(w))
    st_sm, st_ix, st_verb = P.palette_store(enc)
    assert np.array_equal(pw.palette.cpu().numpy(), enc["palette"]), "palette"
    assert np.array_equal(pw.pal_rows.cpu().numpy(), enc["pal_rows"]), "paletted rows"
    assert np.array_equal(pw.verb_rows.cpu().numpy(), enc["verb_rows"]), "verbatim rows"
    assert np.array_equal(pw.sm.cpu().numpy(), st_sm), "sign+mantissa bytes"
    assert np.array_equal(pw.ix.cpu().numpy().view(np.uint32), st_ix), "index words"
    assert np.array_equal(bits(pw.verb), st_verb), "verbatim values"
    return pw, enc


@pytest.mark.parametrize("kind,n,k", [("gauss", 64, 1024), ("gauss", 37, 384), ("few", 50, 640),
                                      ("allverb", 20, 128), ("gauss", 1, 4096), ("gauss", 2500, 896)])
def test_encode_and_decode_bit_exact(kind, n, k):
    sp = need_sp()
    w = _weights(kind, n, k, seed=n + k)
    announce("palette encode", kind, n, k)
    pw, enc = _encode_and_check(w)
    if kind == "few":
        assert pw.n_verb == 0
    if kind == "allverb":
        assert pw.n_pal == 0
    back = sp.palette_decode(pw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(back), W.bf16_bits(w)), "decode is not lossless"


# (m, n, k, kind): m <= 16 -> registers; m > 16 -> rebuilt W + dense GEMM.  K chunks with
# tails of 1, 2 and 3 units of 128 (640, 768, 384, 896, 256) and ragged row counts of both kinds.
GEMM_CASES = [(1, 1, 128, "gauss"), (16, 17, 512, "few"), (2, 1, 256, "allverb"),
              (1, 1000, 640, "gauss"), (3, 300, 768, "gauss"), (16, 37, 384, "gauss"), (5, 257, 896, "few"),
              (2, 40, 256, "allverb"), (1, 4096, 4096, "gauss"), (17, 1000, 640, "gauss"),
              (64, 2048, 1024, "gauss"), (300, 700, 512, "few"), (1, 14336, 4096, "up")]


@pytest.mark.parametrize("m,n,k,kind", GEMM_CASES)
def test_palette_gemm_against_oracle(m, n, k, kind):
    sp = need_sp()
    if kind == "up":
        w, x = W.up_weight(), W.up_x(m)
    else:
        w, x = _weights(kind, n, k, seed=3 * n + k), W.randn_bf16((m, k), seed=m + k)
    announce("palette gemm", kind, m, n, k)
    pw = sp.palette_encode(w.to(DEV))
    y = sp.palette_gemm(x.to(DEV), pw)
    torch.cuda.synchronize()
    ref, mag = P.gemm_ref(W.bf16_bits(x), W.bf16_bits(w))
    assert_within_tolerance(bits(y), ref, mag, "palette gemm %s %dx%dx%d" % (kind, m, n, k))


def test_palette_gemm_repeatable_and_equal_across_calls():
    sp = need_sp()
    m, n, k = 8, 3000, 1024
    w = _weights("gauss", n, k, seed=5)
    x = W.randn_bf16((m, k), seed=6).to(DEV)
    announce("palette gemm repeat", m, n, k)
    pw = sp.palette_encode(w.to(DEV))
    y1 = sp.palette_gemm(x, pw)
    y2 = sp.palette_gemm(x, pw)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
