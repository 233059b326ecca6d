"""sp24_gemm_qx_noalloc (the allocation-free quantise + GEMM) against sp24_gemm_qx.

Both run the same kernels, so outputs and scales must be equal bit for bit.  Two
calls in a row: the first with a larger input (K split over the grid, codes of X
through memory, the two-launch quantiser), the second smaller, so the second
reads a scratch array that still holds the first call's bytes.
"""
import pytest
import torch

sp = pytest.importorskip("bf16_gemm_linear_amd", reason="libsp24.so not built")

pytestmark = pytest.mark.gpu


def _operands(m, n, k, seed):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = (torch.randn(n, k, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    x = torch.randn(m, k, generator=g, device=dev).to(torch.bfloat16)
    values, meta = sp.prune_compress(w)
    qv, sw = sp.quant_fp8(values)
    return x, qv, meta, sw


def _check(m, n, k, seed):
    print("no-alloc case m=%d n=%d k=%d seed=%d plan=%s" % (m, n, k, seed, sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)),
          flush=True)
    x, qv, meta, sw = _operands(m, n, k, seed)
    y_ref, sx_ref = sp.gemm_qx(x, qv, meta, sw)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=x.device)
    sx = torch.full((1,), float("nan"), dtype=torch.float32, device=x.device)
    sp.gemm_qx_noalloc(x, qv, meta, sw, sx, y)
    torch.cuda.synchronize()
    assert torch.equal(sx.view(torch.int32), sx_ref.view(torch.int32))
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_matches_gemm_qx_two_calls_second_smaller():
    big = (64, 4096, 14336)    # split-K over 4 slices + X codes + quantiser partials in the scratch
    small = (16, 14336, 4096)  # X codes through the scratch, one-launch quantiser
    ws_big = sp.workspace_size(sp.OP_GEMM_QX, sp.FP8, *big)
    ws_small = sp.workspace_size(sp.OP_GEMM_QX, sp.FP8, *small)
    assert sp.NOALLOC_SCRATCH_BYTES >= ws_big > ws_small > 0
    _check(*big, seed=7)
    _check(*small, seed=8)


def test_noalloc_single_token_and_ragged():
    # one token: X quantised inside the GEMM kernel, no scratch needed; then a ragged shape
    _check(1, 14336, 4096, seed=9)
    _check(37, 1000, 1152, seed=10)


def test_noalloc_rejects_what_does_not_fit():
    x = torch.zeros(8192, 8192, dtype=torch.bfloat16, device="cuda:0")
    qv = torch.zeros(256, 4096, dtype=torch.uint8, device="cuda:0")
    meta = torch.zeros(256 * 256, dtype=torch.int32, device="cuda:0")
    sw = torch.ones(1, device="cuda:0")
    sx = torch.ones(1, device="cuda:0")
    y = torch.empty(8192, 256, dtype=torch.bfloat16, device="cuda:0")
    need = sp.workspace_size(sp.OP_GEMM_QX, sp.FP8, 8192, 256, 8192)
    assert need > sp.NOALLOC_SCRATCH_BYTES
    with pytest.raises(sp.Sp24Error) as e:
        sp.gemm_qx_noalloc(x, qv, meta, sw, sx, y)
    assert e.value.status == -5
