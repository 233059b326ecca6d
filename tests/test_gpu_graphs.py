"""The library's calls captured in a HIP graph and replayed.

Each case captures one call (buffers allocated before the capture), replays the
graph several times with eager calls of the same kernels and a change of the
input in between, and compares every replay bit for bit with an eager call on
the same input: the quantise + GEMM call fused in one kernel (m = 1), with the
one-launch quantiser (m = 16), with the two-launch quantiser and K split over
four slices (down-projection, m = 64), per token, and the plain sparse GEMM with
its split-K reduction.
"""
import pytest
import torch

sp = pytest.importorskip("bf16_gemm_linear_amd", reason="libsp24.so not built")

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 4


def _weight(n, k, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    values, meta = sp.prune_compress(w)
    qv, sw = sp.quant_fp8(values)
    return qv, meta, sw


def _x(m, k, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(m, k, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _replay_and_compare(m, n, k, make_call, eager):
    """make_call(x, out, scale, ws) issues the call into the given buffers; eager(x)
    returns (y, scale) from a fresh call."""
    print("graph case m=%d n=%d k=%d plan=%s" % (m, n, k, sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)), flush=True)
    x = _x(m, k, seed=m + 1)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    call_bufs = make_call.buffers(m, n, k)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        make_call(x, out, *call_bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make_call(x, out, *call_bufs)
    for r in range(REPLAYS):
        # a new input in the captured buffer, then eager calls of the same kernels
        x.copy_(_x(m, k, seed=100 * r + m, scale=2.0 ** (r - 1)))
        y_ref, s_ref = eager(x)
        other, _ = eager(_x(m, k, seed=7 + r))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_ref.view(torch.int16)), \
            "replay %d differs from the eager call in %d outputs" % (r, int((out != y_ref).sum()))
        assert torch.equal(call_bufs[0].view(torch.int32), s_ref.view(torch.int32)), "replay %d: scale differs" % r
        del other


class _GemmQx:
    def __init__(self, qv, meta, sw):
        self.qv, self.meta, self.sw = qv, meta, sw

    def buffers(self, m, n, k):
        nb = sp.workspace_size(sp.OP_GEMM_QX, sp.FP8, m, n, k)
        return (torch.empty(1, dtype=torch.float32, device=DEV),
                torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV))

    def __call__(self, x, out, scale, ws):
        sp.gemm_qx(x, self.qv, self.meta, self.sw, x_scale=scale, out=out, ws=ws)


class _GemmRowsQx(_GemmQx):
    def buffers(self, m, n, k):
        nb = sp.workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, n, k)
        return (torch.empty(m, dtype=torch.float32, device=DEV),
                torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV))

    def __call__(self, x, out, scales, ws):
        sp.gemm_rows_qx(x, self.qv, self.meta, self.sw, x_scales=scales, out=out, ws=ws)


@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (16, 14336, 4096), (64, 4096, 14336), (1, 4096, 14336)])
def test_gemm_qx_graph_replays_equal_eager(m, n, k):
    qv, meta, sw = _weight(n, k, seed=n + k)
    call = _GemmQx(qv, meta, sw)
    _replay_and_compare(m, n, k, call, lambda x: sp.gemm_qx(x, qv, meta, sw))


@pytest.mark.parametrize("m,n,k", [(1, 4096, 14336), (16, 14336, 4096), (64, 14336, 4096)])
def test_gemm_rows_qx_graph_replays_equal_eager(m, n, k):
    qv, meta, sw = _weight(n, k, seed=n + 3 * k)
    call = _GemmRowsQx(qv, meta, sw)
    _replay_and_compare(m, n, k, call, lambda x: sp.gemm_rows_qx(x, qv, meta, sw))


def test_split_k_gemm_graph_replays_equal_eager():
    m, n, k = 64, 4096, 14336  # K split over 4 slices, partial tiles and the reduction
    plan = sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)
    assert plan["split_k"] > 1
    qv, meta, sw = _weight(n, k, seed=5)
    x = _x(m, k, seed=6)
    xq, sx = sp.quant_fp8(x)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw, out=out, ws=ws)
    for r in range(REPLAYS):
        xq2, sx2 = sp.quant_fp8(_x(m, k, seed=50 + r, scale=1.5))
        xq.copy_(xq2)
        sx.copy_(sx2)
        ref = sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d differs" % r
