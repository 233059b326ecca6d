"""Shared helpers of the GPU parity tests: run the HIP path through the binding
and the oracle on the CPU, on the same seeded inputs, and compare."""
import sys

import numpy as np
import torch

import workloads as W
from oracle import sp24_ref as O

try:  # collection must work on hosts without the built library; GPU tests then fail loudly
    import bf16_gemm_linear_amd as _sp
    _IMPORT_ERROR = None
except ImportError as e:  # pragma: no cover
    _sp, _IMPORT_ERROR = None, e

DEV = torch.device("cuda:0")


def need_sp():
    """The binding; raises if libsp24.so is missing (there is no fallback path)."""
    if _sp is None:
        raise RuntimeError("libsp24.so is not built: %s" % _IMPORT_ERROR)
    return _sp


def announce(*what):
    """Name the case on stdout before its GPU work, so a failing run says which one."""
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor on any device."""
    return W.bf16_bits(t.detach().cpu())


def u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


def f32(t: torch.Tensor) -> np.float32:
    return np.float32(t.detach().cpu().numpy().reshape(-1)[0])


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


class GpuWeight:
    """A weight as the HIP path holds it: compressed (and for FP8 quantised)."""

    def __init__(self, w_bf16_cpu: torch.Tensor, fp8: bool):
        self.n, self.k = w_bf16_cpu.shape
        w = w_bf16_cpu.to(DEV)
        sp = need_sp()
        self.values, self.meta = sp.prune_compress(w)
        del w
        self.fp8 = fp8
        if fp8:
            self.qvalues, self.scale = sp.quant_fp8(self.values)
        else:
            self.qvalues, self.scale = self.values, None


class OracleWeight:
    """The oracle's compressed (and quantised) form of selected rows of a weight.

    Pruning and compression are row-local, so the oracle on a subset of rows
    is exactly its answer for those rows; the FP8 scale is per tensor and is
    computed from every value of the weight (the maximum magnitude survives
    pruning, which the oracle tests pin)."""

    def __init__(self, w_bits: np.ndarray, fp8: bool, rows=None):
        self.rows = np.arange(w_bits.shape[0]) if rows is None else np.asarray(rows)
        self.k = w_bits.shape[1]
        self.values, self.meta = O.prune_compress(w_bits[self.rows])
        self.fp8 = fp8
        if fp8:
            self.scale = O.fp8_scale(w_bits if rows is not None else self.values)
            self.qvalues, _ = O.quant_fp8(self.values, scale=self.scale)
        else:
            self.qvalues, self.scale = self.values, None


def gpu_x(x_bf16_cpu: torch.Tensor, fp8: bool):
    x = x_bf16_cpu.to(DEV)
    if fp8:
        q, s = need_sp().quant_fp8(x)
        return q, s
    return x, None


def oracle_x(x_bits: np.ndarray, fp8: bool):
    if fp8:
        return O.quant_fp8(x_bits)
    return x_bits, None


def oracle_ref(xq, xs, ow: OracleWeight):
    if ow.fp8:
        xh, wh = O.sparse_operands_fp8(xq, xs, ow.qvalues, ow.meta, ow.scale, ow.k)
    else:
        xh, wh = O.sparse_operands_bf16(xq, ow.values, ow.meta, ow.k)
    return O.gemm_ref(xh, wh)


def assert_within_tolerance(y_bits: np.ndarray, ref: np.ndarray, mag: np.ndarray, what=""):
    y = O.bf16_to_f64(y_bits)
    ok = O.within_tolerance(y, ref, mag)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        excess = np.abs(y - ref) / (8e-3 * np.abs(ref) + 1e-4 * mag)
        raise AssertionError(
            "%s: %d of %d outside tolerance; first at %s: y=%r ref=%r mag=%r; worst ratio %.3g"
            % (what, len(bad), ok.size, (int(i), int(j)), y[i, j], ref[i, j], mag[i, j], excess.max()))


def assert_exact_sum_bound(y_bits, ref, mag, what):
    """INT8 paths: the int32 sum is exact, so the only errors are the fp32 scale
    product and the bf16 rounding of the output (2^-8 relative, with 2^-12 for
    the scale product) plus fp32 underflow."""
    y = O.bf16_to_f64(y_bits)
    ok = np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -12) + 2.0 ** -20 * mag
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError("%s: %d outside the exact-sum bound; first at %s: y=%r ref=%r mag=%r"
                             % (what, int((~ok).sum()), (int(i), int(j)), y[i, j], ref[i, j], mag[i, j]))


def full_case(x_cpu, w_cpu, fp8, what, dense=False):
    """Whole pipeline on both sides; compare codes, scales and every output."""
    sp = need_sp()
    announce("gemm", what, "fp8" if fp8 else "bf16", tuple(x_cpu.shape), tuple(w_cpu.shape),
             "dense" if dense else "sparse")
    gw = GpuWeight(w_cpu, fp8)
    xq, xs = gpu_x(x_cpu, fp8)
    if dense:
        wd = sp.decompress(gw.qvalues, gw.meta, gw.k)
        y = sp.dense_gemm(xq, wd, x_scale=xs, w_scale=gw.scale)
    else:
        y = sp.gemm(xq, gw.qvalues, gw.meta, x_scale=xs, w_scale=gw.scale)
    torch.cuda.synchronize()
    ow = OracleWeight(W.bf16_bits(w_cpu), fp8)
    oxq, oxs = oracle_x(W.bf16_bits(x_cpu), fp8)
    assert np.array_equal(u32(gw.meta), O.store_meta(ow.meta))
    if fp8:
        assert f32_bits(f32(gw.scale)) == f32_bits(ow.scale)
        assert f32_bits(f32(xs)) == f32_bits(oxs)
        assert np.array_equal(codes(gw.qvalues), ow.qvalues)
        assert np.array_equal(codes(xq), oxq)
    else:
        assert np.array_equal(bits(gw.values), ow.values)
    ref, mag = oracle_ref(oxq, oxs, ow)
    yb = bits(y)
    assert_within_tolerance(yb, ref, mag, what)
    return y, yb
