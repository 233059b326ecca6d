"""GPU parity of every small-m kernel configuration against the oracle.

The default plan picks one configuration per shape; these tests force each
entry of both configuration tables (SP24_TILE="config,split_k[,rows]") on
shapes that exercise what that configuration's indexing has to get right:
full and partial row blocks, a ragged last row range, a ragged token block,
more K steps than LDS buffers (the ring wraps), fewer steps than buffers,
the K tail of the skinny kernel and the split-K reduction.  Same bar as every
GEMM test: |y - ref| <= 8e-3 |ref| + 1e-4 sum_k |x_k w_k| for every output.
"""
import os
import re

import pytest

import workloads as W
from gpu_helpers import full_case, need_sp

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_SRC = open(os.path.join(ROOT, "bf16_gemm_linear_amd", "csrc", "sp24_internal.hpp")).read()
# stream: id -> (waves along n, row blocks per wave, waves along m, waves along K,
#                token blocks per wave, units per wave per step, buffers)
STREAM = {int(i): tuple(int(v) for v in t) for i, *t in
          re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)", _SRC)}
# skinny: id -> (row blocks, token blocks, waves, batch)
SKINNY = {int(i): tuple(int(v) for v in t) for i, *t in
          re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+)\)", _SRC)}
VARIANTS = [(False, False), (True, False), (False, True), (True, True)]  # (fp8, dense)


def _run(tile, m, n, k, fp8, dense, what, seed):
    sp = need_sp()
    old = os.environ.get("SP24_TILE")
    os.environ["SP24_TILE"] = tile
    try:
        sp.plan(sp.OP_DENSE_GEMM if dense else sp.OP_GEMM, sp.FP8 if fp8 else sp.BF16, m, n, k)
    except sp.Sp24Error:
        pytest.skip("configuration does not fit LDS for this operand type (the planner never picks it)")
    finally:
        if old is None:
            os.environ.pop("SP24_TILE", None)
        else:
            os.environ["SP24_TILE"] = old
    x = W.randn_bf16((m, k), seed=seed)
    w = W.randn_bf16((n, k), seed=seed + 1, std=0.02)
    old = os.environ.get("SP24_TILE")
    os.environ["SP24_TILE"] = tile
    try:
        full_case(x, w, fp8, "%s [SP24_TILE=%s]" % (what, tile), dense=dense)
    finally:
        if old is None:
            os.environ.pop("SP24_TILE", None)
        else:
            os.environ["SP24_TILE"] = old


@pytest.mark.parametrize("fp8,dense", VARIANTS)
@pytest.mark.parametrize("cid", sorted(STREAM))
def test_stream_config_full_rows_ring_wraps(cid, fp8, dense):
    rbw, rb, mw, kw, mb, u, smax = STREAM[cid]
    rows, ups = 16 * rbw * rb, u * kw
    # 3 row ranges (the last one 8 rows), 2 token groups (the last one 5 rows), 9 steps
    m, n, k = 16 * mw * mb + 5, 2 * rows + 8, 128 * ups * 9
    _run("%d,1,%d" % (100 + cid, rows), m, n, k, fp8, dense, "stream %d" % cid, seed=cid * 131)


@pytest.mark.parametrize("fp8,dense", VARIANTS)
@pytest.mark.parametrize("cid", sorted(STREAM))
def test_stream_config_partial_rows_split_k(cid, fp8, dense):
    rbw, rb, mw, kw, mb, u, smax = STREAM[cid]
    ups = u * kw
    # 12-row ranges (the last one 4 rows), 3 tokens, 2 K slices of 1 step each
    m, n, k = 3, 40, 128 * ups * 2
    _run("%d,2,12" % (100 + cid), m, n, k, fp8, dense, "stream %d split" % cid, seed=cid * 131 + 7)


@pytest.mark.parametrize("fp8,dense", VARIANTS)
@pytest.mark.parametrize("cid", sorted(SKINNY))
def test_skinny_config_k_tail(cid, fp8, dense):
    rb, mb, nw, batch = SKINNY[cid]
    # ragged rows and tokens; K = 2 chunks of 512 + a tail of 384, split over 2 slices
    m, n, k = 16 * mb + 3, 16 * rb * 2 + 5, 1408
    _run("%d,2" % cid, m, n, k, fp8, dense, "skinny %d" % cid, seed=cid * 17 + 3)


# The LDS-tiled kernel with its K split over the grid (fp32 partial tiles + the split-K
# reduction): every operand type, ragged m and n, slices of 2 and more steps.
@pytest.mark.parametrize("fp8,dense", VARIANTS)
@pytest.mark.parametrize("m,n,k,sk", [(256, 1000, 1024, 2), (300, 520, 2048, 4), (17, 300, 1024, 4),
                                      (256, 4096, 4096, 8)])
def test_tiled_split_k(m, n, k, sk, fp8, dense):
    _run("99,%d" % sk, m, n, k, fp8, dense, "tiled split-K %dx%dx%d/%d" % (m, n, k, sk), seed=m + n + k + sk)


# The tiled kernel with 128-row tiles (one-byte codes), with and without its K split:
# ragged m and n, one and several tiles of tokens.
@pytest.mark.parametrize("fp8,dense", [v for v in VARIANTS if v[0]])
@pytest.mark.parametrize("m,n,k,sk", [(256, 1000, 1024, 1), (200, 300, 2048, 1), (300, 520, 2048, 2),
                                      (17, 130, 1024, 4), (256, 4096, 4096, 1)])
def test_tiled128(m, n, k, sk, fp8, dense):
    _run("98,%d" % sk, m, n, k, fp8, dense, "tiled 128 rows %dx%dx%d/%d" % (m, n, k, sk), seed=m + n + k + 7 * sk)
