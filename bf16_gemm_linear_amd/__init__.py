"""Python binding of libsp24: 2:4 structured-sparse GEMM for gfx950 (MI355X).

Thin ctypes marshalling over the C ABI declared in include/sp24.h: every call
checks dtypes, devices, shapes and contiguity of torch tensors, passes their
device pointers and the current HIP stream, and raises on a non-OK status.
PyTorch is used only for device memory and streams; all arithmetic runs in the
library's HIP kernels.  If libsp24.so is missing this module raises on import:
there is no fallback.

    values, meta = prune_compress(w)                    # w: [n, k] bf16 on the GPU
    xq, sx = quant_fp8(x)                               # per-tensor dynamic scale
    y = gemm(xq, values_q, meta, x_scale=sx, w_scale=sw)

The operand type follows the tensors: bfloat16, E4M3 codes (torch.uint8 or
torch.float8_e4m3fn) or INT8 codes (torch.int8, from quant_int8).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BF16", "FP8", "INT8", "SCALE_DYNAMIC", "SCALE_STATIC", "OP_GEMM", "OP_QUANT", "OP_DENSE_GEMM", "OP_GEMM_QX",
    "Sp24Error", "lib", "lib_path", "version", "gemm_qx", "gemm_qx_noalloc", "NOALLOC_SCRATCH_BYTES", "quant_fp8_rows", "gemm_rows",
    "slide_prune_pack", "slide_quant_fp8_rows", "slide_quant_int8_rows", "OP_GEMM_ROWS_QX", "gemm_rows_qx",
    "slide_gemm_qx", "OP_GEMM_GROUPS", "quant_fp8_groups", "gemm_groups",
    "quant_int8", "quant_int8_rows", "OP_PALETTE_ANALYZE", "OP_PALETTE_GEMM", "PaletteWeight",
    "palette_encode", "palette_decode", "palette_gemm",
    "prune_compress", "decompress", "quant_fp8", "gemm", "dense_gemm", "workspace_size", "plan",
    "probe_mfma_layout", "probe_mfma_rate", "probe_copy", "probe_read", "probe_ring",
]

BF16, FP8, INT8 = 0, 1, 2
SCALE_DYNAMIC, SCALE_STATIC = 0, 1
OP_GEMM, OP_QUANT, OP_DENSE_GEMM, OP_GEMM_QX, OP_PALETTE_ANALYZE, OP_PALETTE_GEMM = 0, 1, 2, 3, 4, 5
OP_GEMM_ROWS_QX = 6
OP_GEMM_GROUPS = 7

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libsp24.so")

if not os.path.exists(lib_path):
    raise ImportError(
        "libsp24.so is not built (expected at %s); run `python bf16_gemm_linear_amd/build.py`" % lib_path)

lib = ctypes.CDLL(lib_path)

_vp, _i64, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int


class _PaletteStruct(ctypes.Structure):
    """sp24_palette_weight (include/sp24.h)."""
    _fields_ = [("palette", _vp), ("n_pal", _i64), ("sm", _vp), ("ix", _vp), ("pal_rows", _vp),
                ("n_verb", _i64), ("verb", _vp), ("verb_rows", _vp)]


class Plan(ctypes.Structure):
    _fields_ = [("kernel", _int), ("tile_n", _int), ("tile_m", _int), ("waves", _int),
                ("split_k", _int), ("grid_x", _int), ("grid_y", _int), ("grid_z", _int),
                ("config", _int), ("batch", _int), ("workspace_bytes", _sz)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_SIGS = {
    "sp24_prune_compress": [_vp, _i64, _i64, _vp, _vp, _vp],
    "sp24_decompress": [_int, _vp, _vp, _i64, _i64, _vp, _vp],
    "sp24_check_meta": [_vp, _i64, _i64, _vp, _vp],
    "sp24_quant_fp8": [_vp, _i64, _vp, _vp, _int, _vp, _sz, _vp],
    "sp24_quant_int8": [_vp, _i64, _vp, _vp, _int, _vp, _sz, _vp],
    "sp24_gemm": [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_dense_gemm": [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_gemm_qx": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_gemm_qx_noalloc": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "sp24_gemm_rows_qx": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_quant_fp8_groups": [_vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "sp24_gemm_groups": [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_slide_gemm_qx": [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_quant_fp8_rows": [_vp, _i64, _i64, _vp, _vp, _vp],
    "sp24_quant_int8_rows": [_vp, _i64, _i64, _vp, _vp, _vp],
    "sp24_slide_prune_pack": [_vp, _i64, _i64, _int, _vp, _vp],
    "sp24_slide_quant_fp8_rows": [_vp, _i64, _i64, _int, _vp, _vp, _vp],
    "sp24_slide_quant_int8_rows": [_vp, _i64, _i64, _int, _vp, _vp, _vp],
    "sp24_gemm_rows": [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_workspace_size": [_int, _int, _i64, _i64, _i64],
    "sp24_palette_analyze": [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp],
    "sp24_palette_pack": [_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp],
    "sp24_palette_decode": [ctypes.POINTER(_PaletteStruct), _i64, _i64, _vp, _vp],
    "sp24_palette_gemm": [_i64, _i64, _i64, _vp, ctypes.POINTER(_PaletteStruct), _vp, _vp, _sz, _vp],
    "sp24_plan_gemm": [_int, _int, _i64, _i64, _i64, ctypes.POINTER(Plan)],
    "sp24_status_string": [_int],
    "sp24_version": [],
    "sp24_probe_mfma_layout": [_int, _vp, _vp, _vp, _vp, _int, _vp],
    "sp24_probe_mfma_rate": [_int, _int, _int, _int, _vp, _vp],
    "sp24_probe_copy": [_vp, _vp, _sz, _vp],
    "sp24_probe_read": [_vp, _sz, _vp, _vp],
    "sp24_probe_read_blocks": [],
    "sp24_probe_ring": [_int, _int, _int, _int, _vp, _sz, _vp, _sz, _int, _int, _vp, _vp],
}
for _name, _args in _SIGS.items():
    try:
        _f = getattr(lib, _name)
    except AttributeError as _e:
        raise ImportError("%s lacks %s: it was built from older sources; rebuild it with "
                          "`python bf16_gemm_linear_amd/build.py`" % (lib_path, _name)) from _e
    _f.argtypes = _args
    _f.restype = _int
lib.sp24_workspace_size.restype = _sz
lib.sp24_status_string.restype = ctypes.c_char_p


class Sp24Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, lib.sp24_status_string(status).decode(), status))


def _check(fn, status):
    if status != 0:
        raise Sp24Error(fn, status)


def version() -> int:
    return lib.sp24_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must be %d-D" % (name, ndim))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _need_scalar(t, name):
    """A per-tensor scale: at least one fp32 value (the kernels read element 0)."""
    if t.numel() < 1:
        raise ValueError("%s must hold at least one value" % name)


_FP8_T = torch.float8_e4m3fn
_CODE_T = (torch.uint8, torch.float8_e4m3fn)
_ANY_T = (torch.bfloat16, torch.int8) + _CODE_T


def _dtype_of(t):
    """Library dtype of an operand tensor: bf16, int8 codes, else E4M3 codes."""
    return BF16 if t.dtype == torch.bfloat16 else INT8 if t.dtype == torch.int8 else FP8


def _tensor_types(dt):
    """torch dtypes accepted for operands of library dtype `dt`."""
    return torch.bfloat16 if dt == BF16 else torch.int8 if dt == INT8 else _CODE_T


def workspace_size(op: int, dtype: int, m: int, n: int, k: int) -> int:
    return int(lib.sp24_workspace_size(op, dtype, m, n, k))


def plan(op: int, dtype: int, m: int, n: int, k: int) -> dict:
    p = Plan()
    _check("sp24_plan_gemm", lib.sp24_plan_gemm(op, dtype, m, n, k, ctypes.byref(p)))
    return p.as_dict()


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _meta_size(meta: torch.Tensor, n: int, k: int):
    if meta.numel() != max(n * (k // 32), 1):
        raise ValueError("metadata has %d words, expected n * k/32 = %d" % (meta.numel(), n * (k // 32)))


def prune_compress(w: torch.Tensor, values: torch.Tensor | None = None,
                   meta: torch.Tensor | None = None):
    """2:4-prune a bf16 weight [n, k] along k and compress it -> (values [n, k/2], meta).

    `meta` is an int32 tensor of n * k/32 words in the library's storage order:
    the k/32 words of a row are cut into blocks of 4 (128 values of k), and
    block b holds every row's words of that block, row after row.
    """
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    if values is None:
        values = torch.empty(n, k // 2, dtype=torch.bfloat16, device=w.device)
    if meta is None:
        meta = torch.empty(max(n * (k // 32), 1), dtype=torch.int32, device=w.device)
    _need(values, "values", torch.bfloat16, 2, w.device)
    _need(meta, "meta", torch.int32, 1, w.device)
    _meta_size(meta, n, k)
    _check("sp24_prune_compress",
           lib.sp24_prune_compress(_ptr(w), n, k, _ptr(values), _ptr(meta), _stream(w.device)))
    return values, meta


def decompress(values: torch.Tensor, meta: torch.Tensor, k: int, out: torch.Tensor | None = None):
    """Dense pruned W [n, k] from (values, meta); bf16 values give bf16, E4M3 codes give uint8
    codes, INT8 codes give int8 codes."""
    _need(values, "values", _ANY_T, 2)
    _need(meta, "meta", torch.int32, 1, values.device)
    n = values.shape[0]
    _meta_size(meta, n, k)
    dt = _dtype_of(values)
    if out is None:
        t = torch.bfloat16 if dt == BF16 else torch.int8 if dt == INT8 else torch.uint8
        out = torch.empty(n, k, dtype=t, device=values.device)
    _need(out, "out", _tensor_types(dt), 2, values.device)
    _check("sp24_decompress",
           lib.sp24_decompress(dt, _ptr(values), _ptr(meta), n, k, _ptr(out), _stream(values.device)))
    return out


def check_meta(meta: torch.Tensor, k: int, bad: torch.Tensor | None = None) -> torch.Tensor:
    """Count the metadata nibbles that are not a valid kept pair; returns a uint32[1] device
    tensor (`bad`, if given, is added to; otherwise a zeroed one is made)."""
    _need(meta, "meta", torch.int32, 1)
    words = max(k // 32, 1)
    if meta.numel() % words:
        raise ValueError("metadata of %d words does not hold whole rows of k=%d" % (meta.numel(), k))
    if bad is None:
        bad = torch.zeros(1, dtype=torch.int32, device=meta.device)
    _need(bad, "bad", torch.int32, None, meta.device)
    _check("sp24_check_meta",
           lib.sp24_check_meta(_ptr(meta), meta.numel() // words, k, _ptr(bad), _stream(meta.device)))
    return bad


def quant_fp8(x: torch.Tensor, scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, mode: int | None = None):
    """Per-tensor E4M3 quantisation of a bf16 tensor -> (codes uint8, scale fp32[1]).

    mode SCALE_DYNAMIC (the default without `scale`): s = amax/448 is computed on
    the device and written to `scale` (a new fp32[1] tensor when None).
    mode SCALE_STATIC (the default with `scale`): the given fp32 device scalar is used.
    """
    _need(x, "x", torch.bfloat16)
    count = x.numel()
    if mode is None:
        mode = SCALE_DYNAMIC if scale is None else SCALE_STATIC
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, "out", _CODE_T, None, x.device)
    if out.numel() != count:
        raise ValueError("out has the wrong size")
    if scale is None:
        if mode == SCALE_STATIC:
            raise ValueError("static mode needs a scale")
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(scale, "scale", torch.float32, None, x.device)
    _need_scalar(scale, "scale")
    nbytes = workspace_size(OP_QUANT, BF16, count, 1, 1) if mode == SCALE_DYNAMIC else 0
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_quant_fp8",
           lib.sp24_quant_fp8(_ptr(x), count, _ptr(out), _ptr(scale), mode, _ptr(ws), nbytes,
                              _stream(x.device)))
    return out, scale


def quant_int8(x: torch.Tensor, scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, mode: int | None = None):
    """Per-tensor symmetric INT8 quantisation of a bf16 tensor -> (codes int8, scale fp32[1]):
    s = amax/127 (dynamic) or the given device scalar (static), q = clamp(rne(x/s), -127, 127)."""
    _need(x, "x", torch.bfloat16)
    count = x.numel()
    if mode is None:
        mode = SCALE_DYNAMIC if scale is None else SCALE_STATIC
    if out is None:
        out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    _need(out, "out", torch.int8, None, x.device)
    if out.numel() != count:
        raise ValueError("out has the wrong size")
    if scale is None:
        if mode == SCALE_STATIC:
            raise ValueError("static mode needs a scale")
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(scale, "scale", torch.float32, None, x.device)
    _need_scalar(scale, "scale")
    nbytes = workspace_size(OP_QUANT, BF16, count, 1, 1) if mode == SCALE_DYNAMIC else 0
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_quant_int8",
           lib.sp24_quant_int8(_ptr(x), count, _ptr(out), _ptr(scale), mode, _ptr(ws), nbytes,
                               _stream(x.device)))
    return out, scale


def _gemm(sparse, x, w, meta, x_scale, w_scale, out, ws):
    _need(x, "x", _ANY_T, 2)
    dt = _dtype_of(x)
    m, k = x.shape
    _need(w, "w", _tensor_types(dt), 2, x.device)
    n = w.shape[0]
    if sparse:
        _need(meta, "meta", torch.int32, 1, x.device)
        if w.shape[1] * 2 != k:
            raise ValueError("compressed weight shapes do not match k=%d" % k)
        _meta_size(meta, n, k)
    elif w.shape[1] != k:
        raise ValueError("w has %d columns, x has %d" % (w.shape[1], k))
    if dt != BF16:
        if x_scale is None or w_scale is None:
            raise ValueError("FP8 and INT8 operands need x_scale and w_scale")
        _need(x_scale, "x_scale", torch.float32, None, x.device)
        _need(w_scale, "w_scale", torch.float32, None, x.device)
        _need_scalar(x_scale, "x_scale")
        _need_scalar(w_scale, "w_scale")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    op = OP_GEMM if sparse else OP_DENSE_GEMM
    nbytes = workspace_size(op, dt, m, n, k)
    ws = _workspace(nbytes, x.device, ws)
    xs = _ptr(x_scale) if dt != BF16 else None
    wsc = _ptr(w_scale) if dt != BF16 else None
    if sparse:
        st = lib.sp24_gemm(dt, m, n, k, _ptr(x), xs, _ptr(w), _ptr(meta), wsc, _ptr(out), _ptr(ws),
                           nbytes, _stream(x.device))
        _check("sp24_gemm", st)
    else:
        st = lib.sp24_dense_gemm(dt, m, n, k, _ptr(x), xs, _ptr(w), wsc, _ptr(out), _ptr(ws), nbytes,
                                 _stream(x.device))
        _check("sp24_dense_gemm", st)
    return out


def gemm(x, values, meta, x_scale=None, w_scale=None, out=None, ws=None):
    """Y = X . W^T with W compressed 2:4 (values, meta); bf16 output [m, n]."""
    return _gemm(True, x, values, meta, x_scale, w_scale, out, ws)


def quant_fp8_rows(x: torch.Tensor, out: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Per-token E4M3 quantisation of a bf16 X [m, k] (k % 8 == 0) -> (codes uint8 [m, k],
    scales fp32 [m]): row r is quantised with its own dynamic scale amax_r / 448."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    if out is None:
        out = torch.empty(m, k, dtype=torch.uint8, device=x.device)
    _need(out, "out", _CODE_T, 2, x.device)
    if tuple(out.shape) != (m, k):
        raise ValueError("out must be [%d, %d]" % (m, k))
    if scales is None:
        scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(scales, "scales", torch.float32, 1, x.device)
    if scales.numel() != m:
        raise ValueError("scales must hold %d values" % m)
    _check("sp24_quant_fp8_rows", lib.sp24_quant_fp8_rows(_ptr(x), m, k, _ptr(out), _ptr(scales),
                                                          _stream(x.device)))
    return out, scales


def quant_int8_rows(x: torch.Tensor, out: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Per-token INT8 quantisation of a bf16 X [m, k] (k % 8 == 0) -> (codes int8 [m, k],
    scales fp32 [m]): row r is quantised with its own dynamic scale amax_r / 127."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    if out is None:
        out = torch.empty(m, k, dtype=torch.int8, device=x.device)
    _need(out, "out", torch.int8, 2, x.device)
    if tuple(out.shape) != (m, k):
        raise ValueError("out must be [%d, %d]" % (m, k))
    if scales is None:
        scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(scales, "scales", torch.float32, 1, x.device)
    if scales.numel() != m:
        raise ValueError("scales must hold %d values" % m)
    _check("sp24_quant_int8_rows", lib.sp24_quant_int8_rows(_ptr(x), m, k, _ptr(out), _ptr(scales),
                                                            _stream(x.device)))
    return out, scales


def slide_prune_pack(w: torch.Tensor, n_pat: int = 4, out: torch.Tensor | None = None) -> torch.Tensor:
    """SlideSparse load step: prune a bf16 W [n, k] to (2N-2):2N along k and expand it into
    the 2:4 weight W' [n, k (2N-2)/N] (bf16) of N-1 overlapping windows per block of 2N."""
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    kp = k // (2 * n_pat) * 4 * (n_pat - 1)
    if out is None:
        out = torch.empty(n, max(kp, 1), dtype=torch.bfloat16, device=w.device)
    _need(out, "out", torch.bfloat16, 2, w.device)
    _check("sp24_slide_prune_pack", lib.sp24_slide_prune_pack(_ptr(w), n, k, n_pat, _ptr(out),
                                                              _stream(w.device)))
    return out


def slide_quant_fp8_rows(x: torch.Tensor, n_pat: int = 4, out: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None):
    """SlideSparse per-call step: lift a bf16 X [m, k] to the windows of W' and quantise it per
    token -> (codes uint8 [m, k (2N-2)/N], scales fp32 [m])."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    kp = k // (2 * n_pat) * 4 * (n_pat - 1)
    if out is None:
        out = torch.empty(m, max(kp, 1), dtype=torch.uint8, device=x.device)
    _need(out, "out", _CODE_T, 2, x.device)
    if scales is None:
        scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(scales, "scales", torch.float32, 1, x.device)
    _check("sp24_slide_quant_fp8_rows", lib.sp24_slide_quant_fp8_rows(_ptr(x), m, k, n_pat, _ptr(out),
                                                                      _ptr(scales), _stream(x.device)))
    return out, scales


def slide_quant_int8_rows(x: torch.Tensor, n_pat: int = 4, out: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None):
    """As slide_quant_fp8_rows with per-token INT8 codes -> (codes int8 [m, k (2N-2)/N],
    scales fp32 [m], amax/127 per row)."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    kp = k // (2 * n_pat) * 4 * (n_pat - 1)
    if out is None:
        out = torch.empty(m, max(kp, 1), dtype=torch.int8, device=x.device)
    _need(out, "out", torch.int8, 2, x.device)
    if scales is None:
        scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(scales, "scales", torch.float32, 1, x.device)
    _check("sp24_slide_quant_int8_rows", lib.sp24_slide_quant_int8_rows(_ptr(x), m, k, n_pat, _ptr(out),
                                                                        _ptr(scales), _stream(x.device)))
    return out, scales


def gemm_rows(x, values, meta, x_scales, w_scale, out=None, ws=None):
    """Y = X . W^T for E4M3 or INT8 X [m, k] with one scale per row (x_scales fp32 [m], from
    quant_fp8_rows / quant_int8_rows) and compressed weights of the same code type; bf16
    output [m, n]."""
    _need(x, "x", (torch.int8,) + _CODE_T, 2)
    dt = _dtype_of(x)
    m, k = x.shape
    _need(values, "values", _tensor_types(dt), 2, x.device)
    n = values.shape[0]
    if values.shape[1] * 2 != k:
        raise ValueError("compressed weight shapes do not match k=%d" % k)
    _need(meta, "meta", torch.int32, 1, x.device)
    _meta_size(meta, n, k)
    _need(x_scales, "x_scales", torch.float32, 1, x.device)
    if x_scales.numel() != m:
        raise ValueError("x_scales must hold %d values" % m)
    _need(w_scale, "w_scale", torch.float32, None, x.device)
    _need_scalar(w_scale, "w_scale")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    nbytes = workspace_size(OP_GEMM, dt, m, n, k)
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_gemm_rows", lib.sp24_gemm_rows(dt, m, n, k, _ptr(x), _ptr(x_scales), _ptr(values), _ptr(meta),
                                                _ptr(w_scale), _ptr(out), _ptr(ws), nbytes, _stream(x.device)))
    return out


def gemm_qx(x, values, meta, w_scale, x_scale=None, out=None, ws=None):
    """Y = quant_fp8(X) . W^T for a bf16 X [m, k] and E4M3 compressed weights, in one call
    (sp24_gemm_qx): returns (y [m, n] bf16, x_scale fp32[1]), bit-identical to
    quant_fp8 followed by gemm."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    _need(values, "values", _CODE_T, 2, x.device)
    n = values.shape[0]
    if values.shape[1] * 2 != k:
        raise ValueError("compressed weight shapes do not match k=%d" % k)
    _need(meta, "meta", torch.int32, 1, x.device)
    _meta_size(meta, n, k)
    _need(w_scale, "w_scale", torch.float32, None, x.device)
    _need_scalar(w_scale, "w_scale")
    if x_scale is None:
        x_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(x_scale, "x_scale", torch.float32, None, x.device)
    _need_scalar(x_scale, "x_scale")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    nbytes = workspace_size(OP_GEMM_QX, FP8, m, n, k)
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_gemm_qx", lib.sp24_gemm_qx(m, n, k, _ptr(x), _ptr(x_scale), _ptr(values), _ptr(meta),
                                            _ptr(w_scale), _ptr(out), _ptr(ws), nbytes, _stream(x.device)))
    return out, x_scale


def gemm_qx_noalloc(x, values, meta, w_scale, x_scale, out):
    """gemm_qx with the library's own per-GPU scratch array instead of a workspace
    (sp24_gemm_qx_noalloc): the call allocates nothing, so x_scale (fp32[1]) and out
    ([m, n] bf16) must be given.  Bit-identical to gemm_qx.  Calls that may overlap on one
    GPU race on the scratch array; calls on one stream are ordered and safe."""
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    _need(values, "values", _CODE_T, 2, x.device)
    n = values.shape[0]
    if values.shape[1] * 2 != k:
        raise ValueError("compressed weight shapes do not match k=%d" % k)
    _need(meta, "meta", torch.int32, 1, x.device)
    _meta_size(meta, n, k)
    _need(w_scale, "w_scale", torch.float32, None, x.device)
    _need_scalar(w_scale, "w_scale")
    _need(x_scale, "x_scale", torch.float32, None, x.device)
    _need_scalar(x_scale, "x_scale")
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    _check("sp24_gemm_qx_noalloc", lib.sp24_gemm_qx_noalloc(m, n, k, _ptr(x), _ptr(x_scale), _ptr(values),
                                                            _ptr(meta), _ptr(w_scale), _ptr(out),
                                                            _stream(x.device)))
    return out, x_scale


NOALLOC_SCRATCH_BYTES = 32 << 20  # SP24_NOALLOC_SCRATCH_BYTES (include/sp24.h)


def quant_fp8_groups(x: torch.Tensor, group: int, out: torch.Tensor | None = None,
                     scales: torch.Tensor | None = None):
    """E4M3 codes of a bf16 [rows, cols] with one dynamic scale per group of `group`
    consecutive values of a row -> (codes uint8 [rows, cols], scales fp32 [rows, cols/group]).
    For X use the GEMM's group along k; for compressed weights [n, k/2] use group/2."""
    _need(x, "x", torch.bfloat16, 2)
    rows, cols = x.shape
    if group < 8 or group % 8 or cols % group:
        raise ValueError("group must be a multiple of 8 that divides the row length %d" % cols)
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    _need(out, "out", _CODE_T, 2, x.device)
    if tuple(out.shape) != (rows, cols):
        raise ValueError("out must be [%d, %d]" % (rows, cols))
    if scales is None:
        scales = torch.empty(rows, cols // group, dtype=torch.float32, device=x.device)
    _need(scales, "scales", torch.float32, None, x.device)
    if scales.numel() != rows * (cols // group):
        raise ValueError("scales must hold %d values" % (rows * (cols // group)))
    _check("sp24_quant_fp8_groups", lib.sp24_quant_fp8_groups(_ptr(x), rows, cols, group, _ptr(out), _ptr(scales),
                                                              _stream(x.device)))
    return out, scales


def gemm_groups(x, x_scales, values, meta, w_scales, group, out=None, ws=None):
    """Y = X . W^T with E4M3 codes and one scale per group of `group` values of k: X [m, k]
    with x_scales [m, k/group], compressed W codes [n, k/2] with w_scales [n, k/group]
    (quantised in groups of group/2 compressed values); group == k is per-token X and
    per-output-channel W.  bf16 output [m, n]."""
    _need(x, "x", _CODE_T, 2)
    m, k = x.shape
    _need(values, "values", _CODE_T, 2, x.device)
    n = values.shape[0]
    if values.shape[1] * 2 != k:
        raise ValueError("compressed weight shapes do not match k=%d" % k)
    _need(meta, "meta", torch.int32, 1, x.device)
    _meta_size(meta, n, k)
    if group < 128 or group % 128 or k % group:
        raise ValueError("group must be a multiple of 128 that divides k=%d" % k)
    ng = k // group
    _need(x_scales, "x_scales", torch.float32, None, x.device)
    _need(w_scales, "w_scales", torch.float32, None, x.device)
    if x_scales.numel() != m * ng or w_scales.numel() != n * ng:
        raise ValueError("x_scales must hold %d values and w_scales %d" % (m * ng, n * ng))
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    nbytes = workspace_size(OP_GEMM_GROUPS, FP8, m, n, k)
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_gemm_groups", lib.sp24_gemm_groups(m, n, k, group, _ptr(x), _ptr(x_scales), _ptr(values), _ptr(meta),
                                                    _ptr(w_scales), _ptr(out), _ptr(ws), nbytes, _stream(x.device)))
    return out


def _rows_qx_args(x, values, meta, w_scale, kp, x_scales, out):
    _need(x, "x", torch.bfloat16, 2)
    m = x.shape[0]
    _need(values, "values", _CODE_T, 2, x.device)
    n = values.shape[0]
    if values.shape[1] * 2 != kp:
        raise ValueError("compressed weight shapes do not match k=%d" % kp)
    _need(meta, "meta", torch.int32, 1, x.device)
    _meta_size(meta, n, kp)
    _need(w_scale, "w_scale", torch.float32, None, x.device)
    _need_scalar(w_scale, "w_scale")
    if x_scales is None:
        x_scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(x_scales, "x_scales", torch.float32, 1, x.device)
    if x_scales.numel() != m:  # the kernels write one scale per row
        raise ValueError("x_scales must hold %d values" % m)
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if out.shape != (m, n):
        raise ValueError("out must be [%d, %d]" % (m, n))
    return m, n, x_scales, out


def gemm_rows_qx(x, values, meta, w_scale, x_scales=None, out=None, ws=None):
    """Y = X . W^T with X [m, k] bf16 quantised per token inside the call (sp24_gemm_rows_qx):
    returns (y [m, n] bf16, x_scales fp32 [m]), bit-identical to quant_fp8_rows followed by
    gemm_rows."""
    k = x.shape[1] if x.dim() == 2 else 0
    m, n, x_scales, out = _rows_qx_args(x, values, meta, w_scale, k, x_scales, out)
    nbytes = workspace_size(OP_GEMM_ROWS_QX, FP8, m, n, k)
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_gemm_rows_qx", lib.sp24_gemm_rows_qx(m, n, k, _ptr(x), _ptr(x_scales), _ptr(values), _ptr(meta),
                                                      _ptr(w_scale), _ptr(out), _ptr(ws), nbytes,
                                                      _stream(x.device)))
    return out, x_scales


def slide_gemm_qx(x, values, meta, w_scale, n_pat=4, x_scales=None, out=None, ws=None):
    """SlideSparse per call in one call (sp24_slide_gemm_qx): X [m, k] bf16 lifted to the
    windows and quantised per token, times the compressed E4M3 W' [n, k'/2] (k' = k (2N-2)/N);
    returns (y [m, n] bf16, x_scales fp32 [m]), bit-identical to slide_quant_fp8_rows
    followed by gemm_rows."""
    k = x.shape[1] if x.dim() == 2 else 0
    kp = k // (2 * n_pat) * 4 * (n_pat - 1) if 3 <= n_pat <= 8 else 0
    m, n, x_scales, out = _rows_qx_args(x, values, meta, w_scale, kp, x_scales, out)
    nbytes = workspace_size(OP_GEMM_ROWS_QX, FP8, m, n, kp)
    ws = _workspace(nbytes, x.device, ws)
    _check("sp24_slide_gemm_qx", lib.sp24_slide_gemm_qx(n_pat, m, n, k, _ptr(x), _ptr(x_scales), _ptr(values),
                                                        _ptr(meta), _ptr(w_scale), _ptr(out), _ptr(ws), nbytes,
                                                        _stream(x.device)))
    return out, x_scales


class PaletteWeight:
    """A BF16 weight [n, k] in lossless exponent-palette form: a 16-entry exponent palette,
    sign+mantissa bytes and 4-bit indices for the rows whose exponents are all in the
    palette, and the other rows verbatim (see sp24_palette_weight in include/sp24.h)."""

    def __init__(self, n, k, palette, pal_rows, sm, ix, verb_rows, verb):
        self.n, self.k = n, k
        self.palette, self.pal_rows, self.sm, self.ix = palette, pal_rows, sm, ix
        self.verb_rows, self.verb = verb_rows, verb

    @property
    def n_pal(self) -> int:
        return self.pal_rows.numel()

    @property
    def n_verb(self) -> int:
        return self.verb_rows.numel()

    @property
    def nbytes(self) -> int:
        """Bytes of the encoded weight (palette, row lists, bytes, indices, verbatim rows)."""
        return sum(t.numel() * t.element_size() for t in
                   (self.palette, self.pal_rows, self.sm, self.ix, self.verb_rows, self.verb))

    def struct(self) -> _PaletteStruct:
        p = lambda t: t.data_ptr() if t.numel() else None
        return _PaletteStruct(self.palette.data_ptr(), self.n_pal, p(self.sm), p(self.ix), p(self.pal_rows),
                              self.n_verb, p(self.verb), p(self.verb_rows))


def palette_encode(w: torch.Tensor, ws: torch.Tensor | None = None) -> PaletteWeight:
    """Encode a bf16 weight [n, k] (k % 128 == 0): sp24_palette_analyze, one host read of the
    two row counts, then sp24_palette_pack into tensors of the exact (16-row padded) sizes,
    zero-filled so that the padding is defined."""
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    dev = w.device
    pal = torch.empty(16, dtype=torch.uint8, device=dev)
    slot = torch.empty(n, dtype=torch.int32, device=dev)
    counts = torch.empty(2, dtype=torch.int32, device=dev)
    nbytes = workspace_size(OP_PALETTE_ANALYZE, BF16, 0, n, k)
    if nbytes == 0:
        raise ValueError("palette weights need n >= 1 and k % 128 == 0 (got %d x %d)" % (n, k))
    ws = _workspace(nbytes, dev, ws)
    _check("sp24_palette_analyze", lib.sp24_palette_analyze(_ptr(w), n, k, _ptr(pal), _ptr(slot), _ptr(counts),
                                                            _ptr(ws), nbytes, _stream(dev)))
    n_pal, n_verb = (int(v) for v in counts.cpu().tolist())
    pad = lambda r: (r + 15) // 16 * 16
    sm = torch.zeros(pad(n_pal) * k, dtype=torch.uint8, device=dev)
    ix = torch.zeros(pad(n_pal) * k // 8, dtype=torch.int32, device=dev)
    pal_rows = torch.empty(n_pal, dtype=torch.int32, device=dev)
    verb = torch.zeros(pad(n_verb) * k, dtype=torch.bfloat16, device=dev)
    verb_rows = torch.empty(n_verb, dtype=torch.int32, device=dev)
    p = lambda t: _ptr(t) if t.numel() else None
    _check("sp24_palette_pack", lib.sp24_palette_pack(_ptr(w), n, k, _ptr(pal), _ptr(slot), n_pal, n_verb, p(sm),
                                                      p(ix), p(pal_rows), p(verb), p(verb_rows), _stream(dev)))
    return PaletteWeight(n, k, pal, pal_rows, sm, ix, verb_rows, verb)


def palette_decode(pw: PaletteWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    """The bf16 weight [n, k] back from its palette form, bit for bit."""
    dev = pw.palette.device
    if out is None:
        out = torch.empty(pw.n, pw.k, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2, dev)
    st = pw.struct()
    _check("sp24_palette_decode", lib.sp24_palette_decode(ctypes.byref(st), pw.n, pw.k, _ptr(out), _stream(dev)))
    return out


def palette_gemm(x: torch.Tensor, pw: PaletteWeight, out: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . W^T for a bf16 X [m, k] and a palette-form W; bf16 output [m, n].  m <= 16
    rebuilds BF16 in registers; larger m rebuilds W in the workspace and runs the dense GEMM."""
    _need(x, "x", torch.bfloat16, 2, pw.palette.device)
    m, k = x.shape
    if k != pw.k:
        raise ValueError("x has %d columns, the weight %d" % (k, pw.k))
    if out is None:
        out = torch.empty(m, pw.n, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2, x.device)
    if tuple(out.shape) != (m, pw.n):
        raise ValueError("out must be [%d, %d]" % (m, pw.n))
    nbytes = workspace_size(OP_PALETTE_GEMM, BF16, m, pw.n, k)
    ws = _workspace(nbytes, x.device, ws)
    st = pw.struct()
    _check("sp24_palette_gemm", lib.sp24_palette_gemm(m, pw.n, k, _ptr(x), ctypes.byref(st), _ptr(out), _ptr(ws),
                                                      nbytes, _stream(x.device)))
    return out


def dense_gemm(x, w, x_scale=None, w_scale=None, out=None, ws=None):
    """Dense-MFMA baseline Y = X . W^T with an uncompressed W [n, k]."""
    return _gemm(False, x, w, None, x_scale, w_scale, out, ws)


# --------------------------------------------------------------------------- probes

def probe_mfma_layout(variant: int, a: torch.Tensor, b: torch.Tensor, idx: torch.Tensor,
                      c: torch.Tensor, n_exp: int):
    for t, nm in ((a, "a"), (b, "b"), (idx, "idx"), (c, "c")):
        _need(t, nm)
    if a.numel() * a.element_size() < n_exp * 64 * 32 or b.numel() * b.element_size() < n_exp * 64 * 32:
        raise ValueError("a/b too small")
    if idx.numel() * idx.element_size() < n_exp * 64 * 4 or c.numel() * c.element_size() < n_exp * 64 * 64:
        raise ValueError("idx/c too small")
    _check("sp24_probe_mfma_layout",
           lib.sp24_probe_mfma_layout(variant, _ptr(a), _ptr(b), _ptr(idx), _ptr(c), n_exp,
                                      _stream(a.device)))


def probe_mfma_rate(variant: int, iters: int, blocks: int, waves: int, out: torch.Tensor):
    _need(out, "out", torch.float32)
    if out.numel() < blocks * waves * 64:
        raise ValueError("out too small")
    _check("sp24_probe_mfma_rate",
           lib.sp24_probe_mfma_rate(variant, iters, blocks, waves, _ptr(out), _stream(out.device)))


def probe_copy(src: torch.Tensor, dst: torch.Tensor):
    _need(src, "src")
    _need(dst, "dst", None, None, src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check("sp24_probe_copy", lib.sp24_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device)))


def probe_ring(w_kb: int, x_kb: int, stages: int, barrier: bool, w: torch.Tensor, w_stride: int,
               x: torch.Tensor, blocks: int, steps: int, out: torch.Tensor):
    """The GEMM rings' load path without arithmetic (sp24_probe_ring): workgroup b
    reads steps * w_kb KB at w + b * w_stride; x holds one region per XCD (its
    bytes / 8 a power of two)."""
    _need(w, "w")
    _need(x, "x", None, None, w.device)
    _need(out, "out", torch.int32, None, w.device)
    if out.numel() < blocks:
        raise ValueError("out too small")
    if w_kb > 0 and w.numel() * w.element_size() < (blocks - 1) * w_stride + steps * w_kb * 1024:
        raise ValueError("w too small")
    _check("sp24_probe_ring",
           lib.sp24_probe_ring(w_kb, x_kb, stages, 1 if barrier else 0, _ptr(w), w_stride, _ptr(x),
                               x.numel() * x.element_size(), blocks, steps, _ptr(out), _stream(w.device)))


def probe_read(src: torch.Tensor, out: torch.Tensor):
    _need(src, "src")
    _need(out, "out", torch.int32, None, src.device)
    if out.numel() < lib.sp24_probe_read_blocks():
        raise ValueError("out too small")
    _check("sp24_probe_read",
           lib.sp24_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(out), _stream(src.device)))
