"""Host-only checks of libsp24's C ABI: it loads, exports every declared
symbol, validates every argument before any HIP call, and plans launches.

No test here launches a kernel; fake device addresses are only ever passed to
calls that must reject them during validation.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

sp = pytest.importorskip("bf16_gemm_linear_amd", reason="libsp24.so not built")
lib = sp.lib

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EHIP, EMODE, EALIAS = 0, -1, -2, -3, -4, -5, -6, -7, -8
A = 0x7F0000000000  # a 16-byte aligned fake device address (never dereferenced)


def _declared_functions():
    names = []
    for h in ("sp24.h", "sp24_probe.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sp24_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    assert sp.version() == 100
    assert lib.sp24_status_string(0) == b"ok"
    for code in range(-8, 0):
        assert lib.sp24_status_string(code) != b"unknown status"
    assert lib.sp24_status_string(-99) == b"unknown status"


def p(x):
    return ctypes.c_void_p(x)


def gemm(dtype=0, m=8, n=256, k=256, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000,
         wsc=A + 0x400000, y=A + 0x500000, ws=None, wsb=0):
    return lib.sp24_gemm(dtype, m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y), p(ws), wsb, None)


def test_gemm_validation():
    assert gemm(dtype=7) == EDTYPE
    assert gemm(x=None) == ENULL
    assert gemm(meta=None) == ENULL
    assert gemm(dtype=1, xs=None) == ENULL
    assert gemm(m=0) == ESHAPE
    assert gemm(n=0) == ESHAPE
    assert gemm(k=64) == ESHAPE
    assert gemm(k=384 + 32) == ESHAPE
    assert gemm(k=1 << 31) == ESHAPE
    assert gemm(x=A + 8) == EALIGN
    assert gemm(meta=A + 0x300004) == EALIGN
    assert gemm(dtype=1, xs=A + 0x100002) == EALIGN
    assert gemm(y=A + 16) == EALIAS                       # y overlaps x
    assert gemm(y=A + 0x200000 + 32) == EALIAS            # y overlaps values
    assert gemm(dtype=1, y=A + 0x400000 - 64, m=1, n=64) == EALIAS  # y covers w_scale


def test_gemm_workspace_validation():
    # a shape that splits K: small n, long k
    m, n, k = 64, 256, 16384
    need = lib.sp24_workspace_size(0, 1, m, n, k)
    assert need == sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)["workspace_bytes"]
    assert need > 0
    big = 0x10000000
    args = dict(dtype=1, m=m, n=n, k=k, x=A, xs=A + big, w=A + 2 * big, meta=A + 3 * big,
                wsc=A + 4 * big, y=A + 5 * big)
    assert gemm(**args, ws=None, wsb=0) == EWS
    assert gemm(**args, ws=A + 6 * big, wsb=need - 1) == EWS
    assert gemm(**args, ws=A + 6 * big + 4, wsb=need) == EALIGN
    assert gemm(**args, ws=A + 5 * big, wsb=need) == EALIAS


def test_dense_gemm_validation():
    f = lib.sp24_dense_gemm
    assert f(3, 1, 1, 128, p(A), None, p(A + 0x1000), None, p(A + 0x2000), None, 0, None) == EDTYPE
    assert f(0, 1, 1, 100, p(A), None, p(A + 0x1000), None, p(A + 0x2000), None, 0, None) == ESHAPE
    assert f(0, 1, 1, 128, None, None, p(A + 0x1000), None, p(A + 0x2000), None, 0, None) == ENULL
    assert f(1, 1, 1, 128, p(A), None, p(A + 0x1000), None, p(A + 0x2000), None, 0, None) == ENULL


def test_check_meta_validation():
    f = lib.sp24_check_meta
    assert f(None, 4, 64, p(A), None) == ENULL
    assert f(p(A), 4, 64, None, None) == ENULL
    assert f(p(A), 0, 64, p(A + 0x10000), None) == ESHAPE
    assert f(p(A), 4, 48, p(A + 0x10000), None) == ESHAPE
    assert f(p(A + 4), 4, 64, p(A + 0x10000), None) == EALIGN
    assert f(p(A), 4, 64, p(A + 0x10002), None) == EALIGN
    assert f(p(A), 4, 64, p(A + 4), None) == EALIAS


def test_prune_and_decompress_validation():
    f = lib.sp24_prune_compress
    assert f(None, 4, 64, p(A), p(A + 0x1000), None) == ENULL
    assert f(p(A), 0, 64, p(A + 0x10000), p(A + 0x20000), None) == ESHAPE
    assert f(p(A), 4, 48, p(A + 0x10000), p(A + 0x20000), None) == ESHAPE
    assert f(p(A), 4, 64, p(A + 0x10008), p(A + 0x20000), None) == EALIGN
    assert f(p(A), 4, 64, p(A + 256), p(A + 0x20000), None) == EALIAS
    d = lib.sp24_decompress
    assert d(3, p(A), p(A + 0x1000), 4, 64, p(A + 0x2000), None) == EDTYPE
    assert d(0, p(A), None, 4, 64, p(A + 0x2000), None) == ENULL
    assert d(1, p(A), p(A + 0x1000), 4, 16, p(A + 0x2000), None) == ESHAPE
    assert d(1, p(A), p(A + 0x1000), 4, 64, p(A + 0x2004), None) == EALIGN
    assert d(0, p(A), p(A + 0x1000), 4, 64, p(A + 64), None) == EALIAS


@pytest.mark.parametrize("name", ["sp24_quant_fp8", "sp24_quant_int8"])
def test_quant_validation(name):
    f = getattr(lib, name)
    big = 1 << 20
    need = lib.sp24_workspace_size(1, 0, big, 1, 1)
    assert need > 0
    assert lib.sp24_workspace_size(1, 0, 1000, 1, 1) == 0     # small tensors need none
    X, Q, S, W = A, A + 0x1000000, A + 0x2000000, A + 0x3000000
    assert f(p(X), big, p(Q), p(S), 5, p(W), need, None) == EMODE
    assert f(None, big, p(Q), p(S), 0, p(W), need, None) == ENULL
    assert f(p(X), 0, p(Q), p(S), 0, p(W), need, None) == ESHAPE
    assert f(p(X), big, p(Q), p(S), 0, None, 0, None) == EWS
    assert f(p(X), big, p(Q), p(S), 0, p(W), need - 1, None) == EWS
    assert f(p(X + 2), big, p(Q), p(S), 0, p(W), need, None) == EALIGN
    assert f(p(X), big, p(Q), p(S + 1), 0, p(W), need, None) == EALIGN
    assert f(p(X), big, p(X + 16), p(S), 0, p(W), need, None) == EALIAS
    assert f(p(X), big, p(Q), p(Q + 8), 0, p(W), need, None) == EALIAS


def test_plan_table_shapes():
    src = open(os.path.join(ROOT, "bf16_gemm_linear_amd", "csrc", "sp24_internal.hpp")).read()
    table = {int(i): (16 * int(rb), 16 * int(mb), int(nw), int(b)) for i, rb, mb, nw, b in
             re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+)\)", src)}
    stream = {100 + int(i): tuple(int(v) for v in t) for i, *t in
              re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)", src)}
    assert len(table) >= 8 and len(stream) >= 8
    shapes = [(1, 14336, 4096), (16, 14336, 4096), (64, 14336, 4096), (1, 4096, 14336),
              (64, 4096, 14336), (8, 256, 256), (256, 6144, 4096), (256, 4096, 14336),
              (8192, 28672, 8192), (3, 100, 128), (33, 17, 640)]
    for dt in (sp.BF16, sp.FP8):
        for op in (sp.OP_GEMM, sp.OP_DENSE_GEMM):
            for m, n, k in shapes:
                pl = sp.plan(op, dt, m, n, k)
                if pl["kernel"] == 1:   # LDS-tiled: one workgroup per 256 x 256 (or 128 x 256) tile
                    tn = 128 if pl["config"] == 98 else 256
                    assert pl["config"] in (98, 99) and (tn == 256 or dt != sp.BF16)
                    assert (pl["tile_n"], pl["tile_m"], pl["waves"], pl["split_k"]) == (tn, 256, 8, 1)
                    assert pl["grid_x"] == -(-n // tn) * -(-m // 256)
                    continue
                if pl["kernel"] == 2:   # LDS ring: one range of rows per workgroup
                    rbw, rb, mw, kw, mb, u, smax = stream[pl["config"]]
                    assert (pl["tile_m"], pl["waves"], pl["batch"]) == (16 * mw * mb, rbw * mw * kw, u)
                    assert 0 < pl["tile_n"] <= 16 * rbw * rb
                    assert pl["tile_n"] % 4 == 0
                    assert (k // 128) % (pl["split_k"] * u * kw) == 0
                else:
                    assert pl["kernel"] == 0
                    assert table[pl["config"]] == (pl["tile_n"], pl["tile_m"], pl["waves"], pl["batch"])
                assert pl["grid_x"] * pl["tile_n"] >= n and (pl["grid_x"] - 1) * pl["tile_n"] < n
                assert pl["grid_y"] * pl["tile_m"] >= m and (pl["grid_y"] - 1) * pl["tile_m"] < m
                assert pl["grid_z"] == pl["split_k"] >= 1
                ws = pl["workspace_bytes"]
                assert ws == (pl["split_k"] * m * n * 4 if pl["split_k"] > 1 else 0)
                assert lib.sp24_workspace_size(op, dt, m, n, k) == ws


def test_plan_splits_k_only_when_grid_is_small():
    pl = sp.plan(sp.OP_GEMM, sp.FP8, 16, 1024, 16384)   # 64 tiles, 32 chunks of K
    assert pl["split_k"] > 1
    pl = sp.plan(sp.OP_GEMM, sp.FP8, 1, 14336, 4096)    # 896 tiles
    assert pl["split_k"] == 1
    pl = sp.plan(sp.OP_GEMM, sp.FP8, 8, 256, 256)       # one chunk of K: nothing to split
    assert pl["split_k"] == 1


def test_plan_uses_tiled_kernel_for_prefill_only():
    assert sp.plan(sp.OP_GEMM, sp.FP8, 8192, 28672, 8192)["kernel"] == 1
    assert sp.plan(sp.OP_DENSE_GEMM, sp.FP8, 8192, 28672, 8192)["kernel"] == 1
    for m in (1, 16, 64, 256):
        assert sp.plan(sp.OP_GEMM, sp.FP8, m, 14336, 4096)["kernel"] != 1


def test_plan_decode_workgroups_per_cu_by_code_type():
    # m <= 16 with 33-64 rows per CU: one-byte codes take two 8-wave workgroups per CU (512
    # ranges of 28 rows) up to m = 8 and one workgroup of 4 row blocks x 32 tokens above
    # (256 ranges of 56 rows); BF16 -- whose ring for the two-workgroup layout fits a CU's
    # LDS only once -- one workgroup of 4 x 16 rows per CU (256 ranges of 56 rows)
    for m in (1, 4, 8, 16):
        for dt in (sp.FP8, sp.INT8):
            p = sp.plan(sp.OP_GEMM, dt, m, 14336, 4096)
            want = (2, 28, 512, 8) if m <= 8 else (2, 56, 256, 4)
            assert (p["kernel"], p["tile_n"], p["grid_x"], p["waves"]) == want, (m, dt, p)
        p = sp.plan(sp.OP_GEMM, sp.BF16, m, 14336, 4096)
        assert (p["kernel"], p["tile_n"], p["grid_x"], p["config"]) == (2, 56, 256, 113), (m, p)
    # 17-32 rows per CU: one range per CU for every code type
    for dt in (sp.FP8, sp.BF16):
        assert sp.plan(sp.OP_GEMM, dt, 1, 6144, 4096)["grid_x"] == 256


def test_plan_few_rows_per_cu_takes_one_row_block_and_four_k_waves():
    # m <= 16 with at most 16 rows per CU (the down-projection, N = 4096): one 16-row block
    # per workgroup, 256 ranges, 4 waves along K (config 104) for every code type and the
    # dense baseline (the calls that quantise X inside the kernel use 8, config 105)
    for m in (1, 16):
        for dt in (sp.FP8, sp.INT8, sp.BF16):
            p = sp.plan(sp.OP_GEMM, dt, m, 4096, 14336)
            assert (p["kernel"], p["config"], p["tile_n"], p["grid_x"], p["waves"], p["split_k"]) == \
                (2, 104, 16, 256, 4, 1), (m, dt, p)
            assert sp.plan(sp.OP_DENSE_GEMM, dt, m, 4096, 14336)["config"] == 104


def test_plan_tiled_for_wide_layers_at_256_tokens():
    # one tile of tokens and >= 96 tiles (gate+up of an 8B-class layer): BF16 takes the
    # tiled kernel with K split in two (its 256-token stream configurations do not fit
    # LDS); one-byte codes take the tiled kernel with 128-row tiles (224 of them, no
    # split); narrower projections keep the small-m kernels
    for m in (200, 256):
        for dt in (sp.FP8, sp.INT8):
            p8 = sp.plan(sp.OP_GEMM, dt, m, 28672, 4096)
            assert (p8["kernel"], p8["config"], p8["tile_n"], p8["tile_m"]) == (1, 98, 128, 256)
            assert p8["grid_x"] == 224 and p8["split_k"] == 1 and p8["workspace_bytes"] == 0
        p16 = sp.plan(sp.OP_GEMM, sp.BF16, m, 28672, 4096)
        assert p16["kernel"] == 1 and p16["config"] == 99 and p16["split_k"] == 2 and p16["grid_y"] == 2
        assert p16["workspace_bytes"] == 2 * m * 28672 * 4
    for m, n, k in ((256, 6144, 4096), (256, 4096, 4096), (256, 4096, 14336), (128, 28672, 4096)):
        assert sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)["kernel"] == 2, (m, n, k)
    os.environ["SP24_TILE"] = "98,2"
    try:
        with pytest.raises(sp.Sp24Error):   # 128-row tiles take one-byte codes only
            sp.plan(sp.OP_GEMM, sp.BF16, 256, 1024, 1024)
        p = sp.plan(sp.OP_GEMM, sp.FP8, 300, 1000, 1024)
        assert (p["config"], p["tile_n"], p["grid_x"], p["split_k"]) == (98, 128, 8 * 2, 2)
    finally:
        os.environ.pop("SP24_TILE", None)
    for m, n, k in ((256, 6144, 4096), (256, 4096, 4096), (256, 4096, 14336), (128, 28672, 4096),
                    (129, 14336, 4096)):
        assert sp.plan(sp.OP_GEMM, sp.BF16, m, n, k)["kernel"] == 2, (m, n, k)


def test_plan_two_units_per_step_for_sparse_one_byte_codes_at_256_tokens():
    # 128-row workgroups at m = 256 step two units of K (W in whole 128-byte lines) for
    # sparse FP8 / INT8; BF16 (twice the bytes per step) and the dense baseline keep one unit
    for dt in (sp.FP8, sp.INT8):
        qkv = sp.plan(sp.OP_GEMM, dt, 256, 6144, 4096)
        assert (qkv["kernel"], qkv["config"], qkv["tile_n"], qkv["tile_m"], qkv["batch"]) == (2, 129, 96, 64, 2)
        assert (qkv["grid_x"], qkv["grid_y"], qkv["split_k"]) == (64, 4, 1)
        down = sp.plan(sp.OP_GEMM, dt, 256, 4096, 14336)
        assert (down["kernel"], down["config"], down["tile_n"], down["tile_m"], down["batch"]) == (2, 130, 128, 128, 2)
        assert (down["grid_x"], down["grid_y"], down["split_k"]) == (32, 2, 4)
        assert down["workspace_bytes"] == 4 * 256 * 4096 * 4
        assert sp.plan(sp.OP_DENSE_GEMM, dt, 256, 6144, 4096)["config"] == 128
        assert sp.plan(sp.OP_DENSE_GEMM, dt, 256, 4096, 14336)["config"] == 125
    assert sp.plan(sp.OP_GEMM, sp.BF16, 256, 6144, 4096)["config"] == 128
    assert sp.plan(sp.OP_GEMM, sp.BF16, 256, 4096, 14336)["config"] == 125


def test_plan_stream_rows_cover_every_cu_equally():
    # equal row ranges over all 256 CUs: 14336 rows as 512 ranges of 28 (two
    # workgroups per CU), 56 per CU at m = 64, 16 per CU for 4096 rows
    for m, n, k, rows, gx, gz in ((1, 14336, 4096, 28, 512, 1), (64, 14336, 4096, 56, 256, 1),
                                  (1, 4096, 14336, 16, 256, 1), (64, 4096, 14336, 64, 64, 4)):
        pl = sp.plan(sp.OP_GEMM, sp.FP8, m, n, k)
        assert (pl["kernel"], pl["tile_n"], pl["grid_x"], pl["split_k"]) == (2, rows, gx, gz)
        assert (gx * gz) % 256 == 0


def _stream_stage_bytes(dtype, sparse, rbw, rb, mw, kw, mb, u):
    esz = 1 if dtype == sp.FP8 else 2
    ups = u * kw
    wb, mwords, xb = ups * (64 if sparse else 128) * esz, (ups * 4 if sparse else 0), ups * 128 * esz
    return 16 * rbw * rb * (wb + 4 * mwords) + 16 * mw * mb * xb


def test_plan_rejects_stream_configs_that_do_not_fit_lds(monkeypatch):
    # every forced stream configuration plans iff two LDS buffers of its operand type fit
    src = open(os.path.join(ROOT, "bf16_gemm_linear_amd", "csrc", "sp24_internal.hpp")).read()
    stream = {int(i): tuple(int(v) for v in t) for i, *t in
              re.findall(r"X\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)", src)}
    seen = set()
    for cid, (rbw, rb, mw, kw, mb, u, smax) in stream.items():
        k = 128 * u * kw * 4
        monkeypatch.setenv("SP24_TILE", "%d,1" % (100 + cid))
        for dt in (sp.BF16, sp.FP8):
            for op, sparse in ((sp.OP_GEMM, True), (sp.OP_DENSE_GEMM, False)):
                fits = min(smax, 160 * 1024 // _stream_stage_bytes(dt, sparse, rbw, rb, mw, kw, mb, u)) >= 2
                seen.add(fits)
                if fits:
                    assert sp.plan(op, dt, 16 * mw * mb, 16 * rbw * rb * 3, k)["config"] == 100 + cid
                else:
                    with pytest.raises(sp.Sp24Error):
                        sp.plan(op, dt, 16 * mw * mb, 16 * rbw * rb * 3, k)
    assert seen == {True, False}


def test_plan_prefers_the_lds_ring_kernels():
    # every operand type of the decode and layer-sweep shapes plans an LDS-ring kernel (stream
    # or tiled); the skinny kernel is only the fallback for K that no stream step divides
    shapes = [(1, 14336, 4096), (16, 14336, 4096), (64, 14336, 4096), (1, 4096, 14336),
              (64, 4096, 14336), (256, 6144, 4096), (256, 4096, 4096), (256, 28672, 4096),
              (256, 4096, 14336), (200, 28672, 4096), (129, 14336, 4096)]
    for dt in (sp.BF16, sp.FP8):
        for op in (sp.OP_GEMM, sp.OP_DENSE_GEMM):
            for m, n, k in shapes:
                assert sp.plan(op, dt, m, n, k)["kernel"] in (1, 2), (dt, op, m, n, k)


def test_plan_falls_back_to_skinny_kernel_for_odd_k():
    # 31 units of 128 K: the default stream step (2 units) does not divide K
    pl = sp.plan(sp.OP_GEMM, sp.FP8, 1, 14336, 31 * 128)
    assert pl["kernel"] == 0


def test_plan_rejects_what_the_op_rejects():
    with pytest.raises(sp.Sp24Error):
        sp.plan(sp.OP_GEMM, sp.FP8, 1, 1, 100)
    with pytest.raises(sp.Sp24Error):
        sp.plan(sp.OP_QUANT, sp.FP8, 1, 1, 128)
    with pytest.raises(sp.Sp24Error):
        sp.plan(sp.OP_GEMM, 9, 1, 1, 128)


def test_probe_validation():
    assert lib.sp24_probe_mfma_layout(99, p(A), p(A), p(A), p(A), 1, None) == EMODE
    assert lib.sp24_probe_mfma_layout(0, None, p(A), p(A), p(A), 1, None) == ENULL
    assert lib.sp24_probe_mfma_layout(0, p(A), p(A), p(A), p(A), 0, None) == ESHAPE
    assert lib.sp24_probe_mfma_rate(2, 1, 1, 1, p(A), None) == EMODE
    assert lib.sp24_probe_copy(p(A), p(A + 16), 64, None) == EALIAS
    assert lib.sp24_probe_copy(p(A), p(A + 4096), 65, None) == ESHAPE
    assert lib.sp24_probe_read(p(A), 0, p(A + 4096), None) == ESHAPE
    assert lib.sp24_probe_read_blocks() > 0
    # ring probe: arguments checked before any HIP call; shapes outside the built set
    ring = lambda wkb, xkb, st, bar, w=A, ws=64 << 10, x=A + (1 << 24), xb=2 << 20, blocks=4, steps=8, out=A + (1 << 25): \
        lib.sp24_probe_ring(wkb, xkb, st, bar, p(w), ws, p(x), xb, blocks, steps, p(out), None)
    assert ring(8, 16, 4, 1, out=0) == ENULL
    assert ring(8, 16, 4, 1, w=0) == ENULL
    assert ring(8, 16, 4, 1, blocks=0) == ESHAPE
    assert ring(8, 16, 4, 1, ws=8 * 8 * 1024 - 16) == ESHAPE      # region shorter than steps * w_kb KB
    assert ring(8, 16, 4, 1, xb=3 << 20) == ESHAPE                 # x bytes / 8 not a power of two
    assert ring(8, 16, 4, 1, xb=8 * 8 * 1024) == ESHAPE            # region below one step of X
    assert ring(8, 16, 4, 1, ws=(64 << 10) + 8) == EALIGN
    assert ring(16, 16, 4, 1, ws=128 << 10) == EMODE               # not one of SP24_PROBE_RING_SHAPES
    assert ring(8, 16, 5, 1) == EMODE


def gemm_qx(m=8, n=256, k=256, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000,
            wsc=A + 0x400000, y=A + 0x500000, ws=A + 0x600000, wsb=1 << 20):
    return lib.sp24_gemm_qx(m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y), p(ws), wsb, None)


def test_gemm_qx_validation():
    for kw in ("x", "xs", "w", "meta", "wsc", "y"):
        assert gemm_qx(**{kw: None}) == ENULL, kw
    assert gemm_qx(m=0) == ESHAPE
    assert gemm_qx(k=96) == ESHAPE
    assert gemm_qx(x=A + 8) == EALIGN
    assert gemm_qx(meta=A + 0x300004) == EALIGN
    assert gemm_qx(xs=A + 0x100002) == EALIGN
    # the scale output may alias no input and not the output
    assert gemm_qx(xs=A + 0x100) == EALIAS               # inside x (8 x 256 bf16 = 4 KB)
    assert gemm_qx(xs=A + 0x400000) == EALIAS            # the weight scale
    assert gemm_qx(y=A + 0x200000) == EALIAS             # output over the weights
    assert gemm_qx(ws=A + 0x500100) == EALIAS            # workspace over the output


def gemm_qx_noalloc(m=8, n=256, k=256, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000,
                    wsc=A + 0x400000, y=A + 0x500000):
    return lib.sp24_gemm_qx_noalloc(m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y), None)


def test_gemm_qx_noalloc_validation():
    """The allocation-free variant checks its arguments as sp24_gemm_qx does, before any HIP
    call, and rejects shapes whose workspace would exceed its per-GPU scratch array."""
    for kw in ("x", "xs", "w", "meta", "wsc", "y"):
        assert gemm_qx_noalloc(**{kw: None}) == ENULL, kw
    assert gemm_qx_noalloc(m=0) == ESHAPE
    assert gemm_qx_noalloc(k=96) == ESHAPE
    assert gemm_qx_noalloc(x=A + 8) == EALIGN
    assert gemm_qx_noalloc(xs=A + 0x100002) == EALIGN
    assert gemm_qx_noalloc(xs=A + 0x100) == EALIAS
    assert gemm_qx_noalloc(y=A + 0x200000) == EALIAS
    ws_qx = lambda m, n, k: lib.sp24_workspace_size(sp.OP_GEMM_QX, sp.FP8, m, n, k)
    assert sp.NOALLOC_SCRATCH_BYTES == 32 << 20
    # decode shapes fit the scratch array; an 8192-token prefill does not and is refused
    for m, n, k in ((1, 14336, 4096), (64, 14336, 4096), (64, 4096, 14336), (256, 28672, 4096)):
        assert ws_qx(m, n, k) <= sp.NOALLOC_SCRATCH_BYTES, (m, n, k)
    m, n, k = 8192, 28672, 8192
    assert ws_qx(m, n, k) > sp.NOALLOC_SCRATCH_BYTES
    assert gemm_qx_noalloc(m=m, n=n, k=k, x=A, xs=A + (1 << 28), w=A + (2 << 28), meta=A + (4 << 28),
                           wsc=A + (6 << 28), y=A + (8 << 28)) == EWS


def test_groups_validation():
    """sp24_quant_fp8_groups and sp24_gemm_groups check their arguments before any HIP call."""
    qg = lambda x=A, r=4, c=256, g=128, q=A + 0x100000, s=A + 0x200000: lib.sp24_quant_fp8_groups(
        p(x), r, c, g, p(q), p(s), None)
    assert qg(x=None) == ENULL and qg(s=None) == ENULL
    assert qg(g=12) == ESHAPE and qg(c=200) == ESHAPE and qg(r=0) == ESHAPE and qg(g=0) == ESHAPE
    assert qg(x=A + 8) == EALIGN and qg(s=A + 0x200002) == EALIGN
    assert qg(s=A + 0x100) == EALIAS                       # the scales inside X
    gg = lambda m=8, n=256, k=256, g=128, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000, \
        ws_=A + 0x400000, y=A + 0x500000, ws=None, wsb=0: lib.sp24_gemm_groups(
            m, n, k, g, p(x), p(xs), p(w), p(meta), p(ws_), p(y), p(ws), wsb, None)
    for kw in ("x", "xs", "w", "meta", "ws_", "y"):
        assert gg(**{kw: None}) == ENULL, kw
    assert gg(g=64) == ESHAPE and gg(g=384) == ESHAPE and gg(k=96, g=96) == ESHAPE
    assert gg(x=A + 8) == EALIGN and gg(xs=A + 0x100002) == EALIGN
    assert gg(y=A + 0x200000) == EALIAS                     # output over the weights
    assert gg(y=A + 0x100000) == EALIAS                     # output over the X scales
    # a split-K plan without its workspace is refused
    m, n, k = 64, 4096, 14336
    need = lib.sp24_workspace_size(sp.OP_GEMM_GROUPS, sp.FP8, m, n, k)
    assert need > 0
    assert gg(m=m, n=n, k=k, x=A, xs=A + (1 << 24), w=A + (2 << 24), meta=A + (4 << 26), ws_=A + (5 << 26),
              y=A + (6 << 26)) == EWS
    assert lib.sp24_workspace_size(sp.OP_GEMM_GROUPS, sp.BF16, m, n, k) == 0
    # the workspace covers the finer-group plan and the one-group (sp24_gemm) plan
    for m, n, k in ((1, 14336, 4096), (64, 14336, 4096), (16, 4096, 14336), (8192, 28672, 8192)):
        assert lib.sp24_workspace_size(sp.OP_GEMM_GROUPS, sp.FP8, m, n, k) >= \
            lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)


def rows_qx(m=8, n=256, k=256, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000,
            wsc=A + 0x400000, y=A + 0x500000, ws=A + 0x600000, wsb=1 << 20, n_pat=None):
    if n_pat is None:
        return lib.sp24_gemm_rows_qx(m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y), p(ws), wsb, None)
    return lib.sp24_slide_gemm_qx(n_pat, m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y), p(ws), wsb, None)


def test_gemm_rows_qx_and_slide_gemm_qx_validation():
    for n_pat, k in ((None, 256), (4, 1024), (3, 1536)):
        for kw in ("x", "xs", "w", "meta", "wsc", "y"):
            assert rows_qx(n_pat=n_pat, k=k, **{kw: None}) == ENULL, (n_pat, kw)
        assert rows_qx(n_pat=n_pat, k=k, m=0) == ESHAPE
        assert rows_qx(n_pat=n_pat, k=k, x=A + 8) == EALIGN
        assert rows_qx(n_pat=n_pat, k=k, xs=A + 0x100002) == EALIGN
        # the scales (8 x 4 bytes) may alias no input, not the output and not the workspace
        assert rows_qx(n_pat=n_pat, k=k, xs=A + 0x100) == EALIAS
        assert rows_qx(n_pat=n_pat, k=k, xs=A + 0x400000 - 16) == EALIAS   # over the weight scale
        assert rows_qx(n_pat=n_pat, k=k, y=A + 0x200000) == EALIAS
    assert rows_qx(k=96) == ESHAPE
    assert rows_qx(n_pat=2, k=1024) == EMODE and rows_qx(n_pat=9, k=1024) == EMODE
    assert rows_qx(n_pat=4, k=1020) == ESHAPE                  # k % 8 != 0
    assert rows_qx(n_pat=4, k=192) == ESHAPE                   # K' = 288: not a multiple of 128
    assert rows_qx(n_pat=3, k=1028) == ESHAPE                  # k % 6 != 0


def test_gemm_rows_qx_workspace_rule():
    ws_r = lambda m, n, k: lib.sp24_workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, n, k)
    ws_g = lambda m, n, k: lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)
    # decode tokens whose codes fit the kernel's 16 KB: only the GEMM's own workspace
    for m, n, k in ((1, 14336, 4096), (2, 14336, 4096), (4, 14336, 4096), (1, 14336, 6144), (1, 512, 24576)):
        assert ws_r(m, n, k) == (ws_g(m, n, k) + 15) // 16 * 16, (m, n, k)
    # otherwise the codes as well (the per-token quantiser needs no workspace of its own)
    for m, n, k in ((16, 14336, 4096), (64, 14336, 4096), (3, 4096, 14336), (8192, 28672, 8192)):
        assert ws_r(m, n, k) == (ws_g(m, n, k) + 15) // 16 * 16 + (m * k + 15) // 16 * 16, (m, n, k)
    assert ws_r(1, 256, 96) == 0                              # invalid shape
    assert lib.sp24_workspace_size(sp.OP_GEMM_ROWS_QX, sp.BF16, 1, 256, 256) == 0


def test_gemm_qx_workspace_rule():
    ws_qx = lambda m, n, k: lib.sp24_workspace_size(sp.OP_GEMM_QX, sp.FP8, m, n, k)
    ws_g = lambda m, n, k: lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, m, n, k)
    # one decode token (its codes fit the kernel's 16 KB): only the GEMM's own workspace
    for m, n, k in ((1, 14336, 4096), (1, 4096, 14336), (1, 1024, 16384)):
        assert ws_qx(m, n, k) == (ws_g(m, n, k) + 15) // 16 * 16, (m, n, k)
    # larger X: the codes (m*k bytes) and the quantiser's workspace as well
    for m, n, k in ((16, 14336, 4096), (64, 14336, 4096), (16, 4096, 14336), (8192, 28672, 8192)):
        need = lib.sp24_workspace_size(sp.OP_QUANT, sp.BF16, m, 1, k)
        assert ws_qx(m, n, k) == (ws_g(m, n, k) + 15) // 16 * 16 + (m * k + 15) // 16 * 16 + need, (m, n, k)
    assert ws_qx(1, 256, 96) == 0                         # invalid shape
    assert lib.sp24_workspace_size(sp.OP_GEMM_QX, sp.BF16, 1, 256, 256) == 0  # FP8 only
    # a workspace too small is rejected before any launch
    m, n, k = 64, 14336, 4096
    assert gemm_qx(m=m, n=n, k=k, x=A, xs=A + (1 << 24), w=A + (2 << 24), meta=A + (4 << 26),
                   wsc=A + (6 << 26), y=A + (7 << 26), ws=A + (8 << 26), wsb=ws_qx(m, n, k) - 16) == EWS


@pytest.mark.parametrize("name", ["sp24_quant_fp8_rows", "sp24_quant_int8_rows"])
def test_quant_rows_validation(name):
    f = lambda x=A, m=4, k=256, q=A + 0x100000, s=A + 0x200000: getattr(lib, name)(
        p(x), m, k, p(q), p(s), None)
    assert f(x=None) == ENULL and f(q=None) == ENULL and f(s=None) == ENULL
    assert f(m=0) == ESHAPE and f(k=0) == ESHAPE and f(k=12) == ESHAPE
    assert f(x=A + 8) == EALIGN and f(q=A + 0x100008) == EALIGN and f(s=A + 0x200002) == EALIGN
    assert f(q=A + 0x400) == EALIAS                       # codes over X (4 x 256 bf16 = 2 KB)
    assert f(s=A + 0x10) == EALIAS                        # scales over X
    assert f(s=A + 0x100010) == EALIAS                    # scales over the codes


@pytest.mark.parametrize("dtype", [1, 2])
def test_gemm_rows_validation(dtype):
    g = lambda m=8, n=256, k=256, x=A, xs=A + 0x100000, w=A + 0x200000, meta=A + 0x300000, wsc=A + 0x400000, \
        y=A + 0x500000, dt=dtype: lib.sp24_gemm_rows(dt, m, n, k, p(x), p(xs), p(w), p(meta), p(wsc), p(y),
                                                     None, 0, None)
    assert g(dt=0) == EDTYPE and g(dt=3) == EDTYPE          # codes with scales only
    assert g(xs=None) == ENULL and g(wsc=None) == ENULL and g(meta=None) == ENULL
    assert g(k=96) == ESHAPE
    assert g(xs=A + 0x100002) == EALIGN
    # the output may not overlap any of the m row scales (m * 4 bytes)
    assert g(xs=A + 0x500000 - 16, m=8) == EALIAS


def test_slide_validation():
    pk = lambda w=A, n=4, k=64, np_=4, out=A + 0x100000: lib.sp24_slide_prune_pack(p(w), n, k, np_, p(out), None)
    assert pk(w=None) == ENULL and pk(out=None) == ENULL
    assert pk(np_=2) == EMODE and pk(np_=9) == EMODE
    assert pk(k=60) == ESHAPE and pk(n=0) == ESHAPE
    assert pk(w=A + 4) == EALIGN
    assert pk(out=A + 0x100) == EALIAS
    for fn in (lib.sp24_slide_quant_fp8_rows, lib.sp24_slide_quant_int8_rows):
        qz = lambda x=A, m=2, k=64, np_=4, q=A + 0x100000, s=A + 0x200000: fn(p(x), m, k, np_, p(q), p(s), None)
        assert qz(x=None) == ENULL and qz(s=None) == ENULL
        assert qz(np_=1) == EMODE
        assert qz(k=60) == ESHAPE and qz(k=36, np_=3) == ESHAPE     # 36 % 8 != 0
        assert qz(q=A + 8) == EALIGN
        assert qz(s=A + 0x10) == EALIAS


def test_int8_validation_and_plan():
    # INT8 carries scales like FP8 and has the same plans (one-byte codes)
    assert gemm(dtype=2, xs=None) == ENULL
    assert gemm(dtype=2, wsc=None) == ENULL
    assert gemm(dtype=2, xs=A + 0x100002) == EALIGN
    assert gemm(dtype=2, y=A + 0x400000 - 64, m=1, n=64) == EALIAS
    # exact int32 sums: k is limited to 131072
    assert gemm(dtype=2, k=131072 + 128, x=A, y=A + (1 << 36)) == ESHAPE
    pl = sp.Plan()
    assert lib.sp24_plan_gemm(sp.OP_GEMM, sp.INT8, 8, 256, 131072 + 128, ctypes.byref(pl)) == ESHAPE
    assert lib.sp24_plan_gemm(sp.OP_GEMM, sp.INT8, 8, 256, 131072, ctypes.byref(pl)) == OK
    assert lib.sp24_plan_gemm(sp.OP_GEMM, sp.FP8, 8, 256, 131072 + 128, ctypes.byref(pl)) == OK
    for m, n, k in ((1, 14336, 4096), (16, 4096, 14336), (64, 28672, 8192), (8192, 28672, 8192), (600, 32771, 384)):
        for op in (sp.OP_GEMM, sp.OP_DENSE_GEMM):
            assert sp.plan(op, sp.INT8, m, n, k) == sp.plan(op, sp.FP8, m, n, k), (op, m, n, k)
            assert lib.sp24_workspace_size(op, 2, m, n, k) == lib.sp24_workspace_size(op, 1, m, n, k)
    f = lib.sp24_dense_gemm
    assert f(2, 1, 1, 128, p(A), None, p(A + 0x1000), None, p(A + 0x2000), None, 0, None) == ENULL
    assert lib.sp24_workspace_size(sp.OP_GEMM_QX, 2, 1, 256, 256) == 0   # FP8 only


def _pw(palette=A, n_pal=3, sm=A + 0x10000, ix=A + 0x20000, pal_rows=A + 0x30000, n_verb=1, verb=A + 0x40000,
        verb_rows=A + 0x50000):
    return sp._PaletteStruct(palette, n_pal, sm, ix, pal_rows, n_verb, verb, verb_rows)


def test_palette_analyze_and_pack_validation():
    n, k = 4, 128
    need = lib.sp24_workspace_size(sp.OP_PALETTE_ANALYZE, 0, 0, n, k)
    assert need >= 256 * 4 + 256 + n * 4
    assert lib.sp24_workspace_size(sp.OP_PALETTE_ANALYZE, 0, 0, n, 12) == 0     # k % 8
    an = lambda w=A, n=n, k=k, pal=A + 0x10000, slot=A + 0x20000, cnt=A + 0x30000, ws=A + 0x40000, wsb=need: \
        lib.sp24_palette_analyze(p(w), n, k, p(pal), p(slot), p(cnt), p(ws), wsb, None)
    assert an(w=None) == ENULL and an(pal=None) == ENULL and an(slot=None) == ENULL and an(cnt=None) == ENULL
    assert an(n=0) == ESHAPE and an(k=12) == ESHAPE and an(k=0) == ESHAPE and an(k=64) == ESHAPE
    assert an(w=A + 8) == EALIGN and an(pal=A + 0x10004) == EALIGN and an(slot=A + 0x20002) == EALIGN
    assert an(ws=None) == EWS and an(wsb=need - 1) == EWS and an(ws=A + 0x40008) == EALIGN
    assert an(pal=A + 0x100) == EALIAS                      # palette inside W (4 x 128 bf16 = 1 KB)
    assert an(slot=A + 0x10000) == EALIAS                   # slots over the palette
    pk = lambda w=A, n=n, k=k, pal=A + 0x10000, slot=A + 0x20000, npl=3, nvb=1, sm=A + 0x30000, ix=A + 0x40000, \
        pr=A + 0x50000, vb=A + 0x60000, vr=A + 0x70000: lib.sp24_palette_pack(
            p(w), n, k, p(pal), p(slot), npl, nvb, p(sm), p(ix), p(pr), p(vb), p(vr), None)
    assert pk(npl=2) == ESHAPE and pk(npl=-1, nvb=5) == ESHAPE   # n_pal + n_verb == n
    assert pk(sm=None) == ENULL and pk(vr=None) == ENULL
    assert pk(w=A + 4) == EALIGN and pk(sm=A + 0x30008) == EALIGN and pk(pr=A + 0x50002) == EALIGN
    assert pk(sm=A + 0x100) == EALIAS                        # codes over W
    assert pk(ix=A + 0x30000 + 64) == EALIAS                 # indices over the codes (16 x 128 bytes)


def test_palette_decode_and_gemm_validation():
    n, k = 4, 128
    d = lambda pw=None, n=n, k=k, out=A + 0x100000: lib.sp24_palette_decode(
        ctypes.byref(pw if pw is not None else _pw()), n, k, p(out), None)
    assert lib.sp24_palette_decode(None, n, k, p(A + 0x100000), None) == ENULL
    assert d(out=None) == ENULL
    assert d(pw=_pw(palette=None)) == ENULL
    assert d(pw=_pw(n_pal=2)) == ESHAPE                      # rows do not add up to n
    assert d(pw=_pw(sm=None)) == ENULL and d(pw=_pw(verb_rows=None)) == ENULL
    assert d(pw=_pw(palette=A + 8)) == EALIGN and d(pw=_pw(ix=A + 0x20004)) == EALIGN
    assert d(pw=_pw(pal_rows=A + 0x30002)) == EALIGN
    assert d(k=12) == ESHAPE
    assert d(out=A + 0x40000 + 64) == EALIAS                 # output over the verbatim rows
    # n_pal == 0: its arrays may be NULL (the verbatim ones are still checked)
    assert d(pw=_pw(n_pal=0, n_verb=4, sm=None, ix=None, pal_rows=None), out=A + 8) == EALIGN
    g = lambda m=1, n=n, k=k, x=A + 0x200000, pw=None, y=A + 0x300000, ws=None, wsb=0: lib.sp24_palette_gemm(
        m, n, k, p(x), ctypes.byref(pw if pw is not None else _pw()), p(y), p(ws), wsb, None)
    assert g(x=None) == ENULL and g(y=None) == ENULL
    assert g(k=64) == ESHAPE and g(m=0) == ESHAPE and g(pw=_pw(n_verb=3)) == ESHAPE
    assert g(x=A + 0x200008) == EALIGN
    assert g(y=A + 0x200000 + 64) == EALIAS                  # y over x
    assert g(y=A + 0x10000) == EALIAS                        # y over the codes
    # m <= 16 needs no workspace; larger m needs the rebuilt weight plus the dense GEMM's
    assert lib.sp24_workspace_size(sp.OP_PALETTE_GEMM, 0, 16, 4096, 4096) == 0
    big = lib.sp24_workspace_size(sp.OP_PALETTE_GEMM, 0, 17, 4096, 4096)
    assert big >= 4096 * 4096 * 2
    assert lib.sp24_workspace_size(sp.OP_PALETTE_GEMM, 0, 17, 4096, 4000) == 0   # k % 128
    assert g(m=17, n=4, ws=None) == EWS


def test_tiled_split_k_plan(monkeypatch):
    """The tiled kernel's K split (SP24_TILE="99,split"): whole, even numbers of K steps per
    slice, the fp32 partials in the workspace; other splits are rejected."""
    monkeypatch.setenv("SP24_TILE", "99,4")
    pl = sp.plan(sp.OP_GEMM, sp.FP8, 256, 4096, 4096)
    assert pl["kernel"] == 1 and pl["split_k"] == 4 and pl["grid_y"] == 4
    assert pl["workspace_bytes"] == 4 * 256 * 4096 * 4
    assert lib.sp24_workspace_size(sp.OP_GEMM, sp.FP8, 256, 4096, 4096) == pl["workspace_bytes"]
    for dt, k, split in ((sp.FP8, 1024, 3), (sp.FP8, 1024, 8), (sp.BF16, 1024, 16), (sp.INT8, 384, 2)):
        monkeypatch.setenv("SP24_TILE", "99,%d" % split)   # 8 steps of 128 in 3 or in 8 (odd), 16 of 64 in 16, 3 in 2
        with pytest.raises(sp.Sp24Error):
            sp.plan(sp.OP_GEMM, dt, 256, 512, k)
    monkeypatch.setenv("SP24_TILE", "99,2")
    assert sp.plan(sp.OP_GEMM, sp.BF16, 256, 512, 1024)["split_k"] == 2
