"""Thin Python binding of ``libarnfp8.so``, the gfx950 fused all-reduce epilogue.

Every entry point here has the C ABI's name and argument order and does only
argument marshalling: tensors are checked to be dense device memory of the
declared element type and of the size the call's shape implies (the library
sees bare pointers and cannot), then become device pointers; the stream
becomes the current PyTorch stream's handle; a non-zero status raises
``ArnFp8Error``.
All arithmetic runs in the library's HIP kernels; there is no CPU fallback --
if the library is not built, every call raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "ArnFp8Error", "MAX_P", "MAX_COLS", "STATUS",
    "arnfp8_run", "arnfp8_run_ex", "arn_sum_bf16", "arnfp8_status_string", "Launch",
    "library", "library_path", "VARIANT_AUTO", "VARIANT_ROW", "arnfp8_stage_bytes",
    "arnfp8_run_share", "SIMD_WIDTH", "arnfp8_run_fmt", "FMT_E4M3FN", "FMT_E5M2", "FMT_MXFP8",
    "CVT_BF16", "arnfp8_convert_f32", "STORES_AUTO", "STORES_NT", "STORES_SC1",
    "SplitOpts", "arnfp8_split_workspace_bytes", "arnfp8_split_parts", "arnfp8_run_split",
    "arnfp8_run_split_noalloc",
    "NOALLOC_MAX_ROWS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libarnfp8.so")

MAX_P = 8
MAX_COLS = 65536
NOALLOC_MAX_ROWS = 4096  # rows of the allocation-free split call (ARNFP8_NOALLOC_MAX_ROWS)
STATUS = {
    0: "ARNFP8_OK", 1: "ARNFP8_NULL_POINTER", 2: "ARNFP8_MISALIGNED", 3: "ARNFP8_BAD_SHAPE",
    4: "ARNFP8_BAD_P", 5: "ARNFP8_ALIAS", 6: "ARNFP8_HIP_ERROR", 7: "ARNFP8_BAD_CONFIG",
    8: "ARNFP8_BAD_SHARE", 9: "ARNFP8_BAD_FORMAT", 10: "ARNFP8_BAD_SCALAR",
    11: "ARNFP8_BAD_WORKSPACE",
}
FMT_E4M3FN = 0
FMT_E5M2 = 1
FMT_MXFP8 = 2
CVT_BF16 = 16
SIMD_WIDTH = 16


class ArnFp8Error(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({arnfp8_status_string(status)})")


VARIANT_AUTO = 0
VARIANT_ROW = 1


class Launch(ctypes.Structure):
    """``arnfp8_launch``: launch options; 0 in a field means automatic."""

    _fields_ = [("variant", ctypes.c_int), ("threads", ctypes.c_int), ("vpt", ctypes.c_int),
                ("grid", ctypes.c_int), ("stores", ctypes.c_int)]


STORES_AUTO = 0
STORES_NT = 1
STORES_SC1 = 2


class SplitOpts(ctypes.Structure):
    """``arnfp8_split_opts``: parts per row (0: automatic) and the bound of the
    wait for a partner's partial (0: default; -1: none, the fallback alone)."""

    _fields_ = [("parts", ctypes.c_int), ("spin_polls", ctypes.c_int)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load ``libarnfp8.so`` (built in-tree by ``all_reduce_rmsnorm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is not built; run `python -m all_reduce_rmsnorm_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.arnfp8_run.restype = ctypes.c_int
        L.arnfp8_run.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, vp, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_float, i64, i64, ctypes.c_int, vp]
        L.arnfp8_run_ex.restype = ctypes.c_int
        L.arnfp8_run_ex.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, vp, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_float, i64, i64, ctypes.c_int, vp,
                                    ctypes.POINTER(Launch)]
        L.arnfp8_run_fmt.restype = ctypes.c_int
        L.arnfp8_run_fmt.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, vp, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_float, i64, i64, ctypes.c_int,
                                     ctypes.c_int, vp, ctypes.POINTER(Launch)]
        L.arnfp8_convert_f32.restype = ctypes.c_int
        L.arnfp8_convert_f32.argtypes = [vp, vp, i64, ctypes.c_int, vp]
        L.arnfp8_stage_bytes.restype = ctypes.c_int64
        L.arnfp8_stage_bytes.argtypes = [i64, i64, ctypes.c_int]
        L.arnfp8_run_share.restype = ctypes.c_int
        L.arnfp8_run_share.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, i64, i64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, vp]
        L.arnfp8_split_workspace_bytes.restype = ctypes.c_int64
        L.arnfp8_split_workspace_bytes.argtypes = [i64]
        L.arnfp8_split_parts.restype = ctypes.c_int
        L.arnfp8_split_parts.argtypes = [i64, i64]
        L.arnfp8_run_split.restype = ctypes.c_int
        L.arnfp8_run_split.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, vp, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, i64, i64, ctypes.c_int,
                                       vp, i64, vp, ctypes.POINTER(SplitOpts)]
        L.arnfp8_run_split_noalloc.restype = ctypes.c_int
        L.arnfp8_run_split_noalloc.argtypes = [ctypes.POINTER(vp), vp, vp, vp, vp, vp,
                                               ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                               i64, i64, ctypes.c_int, vp,
                                               ctypes.POINTER(SplitOpts)]
        L.arn_sum_bf16.restype = ctypes.c_int
        L.arn_sum_bf16.argtypes = [ctypes.POINTER(vp), vp, i64, i64, ctypes.c_int, vp]
        L.arnfp8_status_string.restype = ctypes.c_char_p
        L.arnfp8_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


_BF16 = ("bfloat16",)
_FP8 = ("float8_e4m3fn", "float8_e5m2", "uint8", "int8")
_F32 = ("float32",)
_U8 = ("uint8", "int8")


def _ptr(t, kinds=None, what="tensor", nbytes=None):
    """Address of a tensor's data (or a raw integer address, or None).

    Tensors must be dense (contiguous), of one of the dtypes in ``kinds`` when
    it is given, and hold at least ``nbytes`` bytes when that is positive: the
    library reads and writes plain row-major memory of the sizes the call's
    shape implies.  ``_on_device`` checks where they live.
    """
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (the library reads dense row-major memory)")
    if kinds is not None and str(t.dtype).replace("torch.", "") not in kinds:
        raise TypeError(f"{what} has dtype {t.dtype}; expected one of {', '.join(kinds)}")
    if nbytes is not None and nbytes > 0 and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes; the call's shape "
                         f"needs {nbytes}")
    return t.data_ptr()


def _ptr_array(inputs, nbytes=None):
    ptrs = [_ptr(x, _BF16, f"inputs[{i}]", nbytes) for i, x in enumerate(inputs)]
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)


def _on_device(**tensors):
    """Every tensor argument (lists included) must be device memory."""
    for what, t in tensors.items():
        items = list(enumerate(t)) if isinstance(t, (list, tuple)) else [(None, t)]
        for i, x in items:
            if x is None or isinstance(x, int):
                continue
            if x.device.type != "cuda":
                name = what if i is None else f"{what}[{i}]"
                raise ValueError(f"{name} must be a device (cuda) tensor, got {x.device}")


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shape(inputs, rows, cols, P):
    if P is None:
        P = len(inputs)
    if (rows is None or cols is None) and len(inputs) > 0 and hasattr(inputs[0], "shape"):
        shp = inputs[0].shape
        if cols is None:
            cols = int(shp[-1])
        if rows is None:
            rows = int(inputs[0].numel() // shp[-1]) if shp[-1] else 0
    return int(rows), int(cols), int(P)


def arnfp8_status_string(status: int) -> str:
    return library().arnfp8_status_string(int(status)).decode()


def arnfp8_run(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps, weight_offset,
               scale_ub, rows=None, cols=None, P=None, stream=None) -> None:
    """The fused epilogue (sum, residual, RMSNorm, per-row e4m3fn quant), one launch.

    ``inputs``: sequence of P bf16 [rows, cols] device tensors in rank order.
    ``residual_in`` / ``residual_out``: bf16 [rows, cols] or None (may be the same tensor).
    ``out_fp8``: e4m3fn (or uint8) [rows, cols]; ``scales``: fp32 [rows] or [rows, 1];
    ``gamma``: bf16 [cols].  ``rows``, ``cols``, ``P`` default to the inputs' shape.
    Runs on ``stream`` (default: PyTorch's current stream).
    """
    rows, cols, P = _shape(inputs, rows, cols, P)
    n = rows * cols
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(out_fp8, _FP8, "out_fp8", n),
            _ptr(scales, _F32, "scales", 4 * rows), _ptr(gamma, _BF16, "gamma", 2 * cols))
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               out_fp8=out_fp8, scales=scales, gamma=gamma)
    st = library().arnfp8_run(*ptrs, float(eps), float(weight_offset), float(scale_ub), rows,
                              cols, P, _stream(stream))
    if st != 0:
        raise ArnFp8Error("arnfp8_run", st)


def arnfp8_run_ex(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps, weight_offset,
                  scale_ub, rows=None, cols=None, P=None, stream=None, launch=None) -> None:
    """``arnfp8_run`` with explicit launch options (a ``Launch``, a dict of its
    fields, or None for automatic)."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    if isinstance(launch, dict):
        launch = Launch(**launch)
    opt = ctypes.byref(launch) if launch is not None else None
    n = rows * cols
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(out_fp8, _FP8, "out_fp8", n),
            _ptr(scales, _F32, "scales", 4 * rows), _ptr(gamma, _BF16, "gamma", 2 * cols))
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               out_fp8=out_fp8, scales=scales, gamma=gamma)
    st = library().arnfp8_run_ex(*ptrs, float(eps), float(weight_offset), float(scale_ub), rows,
                                 cols, P, _stream(stream), opt)
    if st != 0:
        raise ArnFp8Error("arnfp8_run_ex", st)


def arn_sum_bf16(inputs, out, rows=None, cols=None, P=None, stream=None) -> None:
    """Rank-order fp32 sum of P bf16 slabs, rounded once to bf16, into ``out``."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    n = rows * cols
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(out, _BF16, "out", 2 * n))
    _on_device(inputs=inputs, out=out)
    st = library().arn_sum_bf16(*ptrs, rows, cols, P, _stream(stream))
    if st != 0:
        raise ArnFp8Error("arn_sum_bf16", st)


def arnfp8_stage_bytes(rows: int, cols: int, ngpus: int) -> int:
    """Bytes of one rank's staging slot in the two-stage layout (-1 if invalid)."""
    return int(library().arnfp8_stage_bytes(int(rows), int(cols), int(ngpus)))


def arnfp8_run_share(inputs, residual_in, residual_out, staging, gamma, eps, weight_offset,
                     scale_ub, rows=None, cols=None, P=None, ngpus=1, rank=0, stream=None) -> None:
    """The fused epilogue on rank ``rank``'s row share, fp8 rows + scales into ``staging``."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    n = rows * cols
    slot = arnfp8_stage_bytes(rows, cols, ngpus) if rows >= 0 and cols > 0 and ngpus >= 1 else None
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(staging, _U8, "staging", slot),
            _ptr(gamma, _BF16, "gamma", 2 * cols))
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               staging=staging, gamma=gamma)
    st = library().arnfp8_run_share(*ptrs, float(eps), float(weight_offset), float(scale_ub),
                                    rows, cols, P, int(ngpus), int(rank), _stream(stream))
    if st != 0:
        raise ArnFp8Error("arnfp8_run_share", st)


def arnfp8_run_fmt(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps, weight_offset,
                   scale_ub, out_format=FMT_E4M3FN, rows=None, cols=None, P=None, stream=None,
                   launch=None) -> None:
    """The fused epilogue with output format ``out_format`` (FMT_E4M3FN,
    FMT_E5M2: fp32 per-row ``scales``; FMT_MXFP8: uint8 E8M0 ``scales``
    [rows, cols / 32])."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    if isinstance(launch, dict):
        launch = Launch(**launch)
    opt = ctypes.byref(launch) if launch is not None else None
    # an unknown format is left to the library, which reports it as BAD_FORMAT
    scale_kinds = {FMT_MXFP8: _U8, FMT_E4M3FN: _F32, FMT_E5M2: _F32}.get(int(out_format))
    n = rows * cols
    scale_bytes = {FMT_MXFP8: rows * (cols // 32), FMT_E4M3FN: 4 * rows,
                   FMT_E5M2: 4 * rows}.get(int(out_format))
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(out_fp8, _FP8, "out_fp8", n),
            _ptr(scales, scale_kinds, "scales", scale_bytes), _ptr(gamma, _BF16, "gamma", 2 * cols))
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               out_fp8=out_fp8, scales=scales, gamma=gamma)
    st = library().arnfp8_run_fmt(*ptrs, float(eps), float(weight_offset), float(scale_ub), rows,
                                  cols, P, int(out_format), _stream(stream), opt)
    if st != 0:
        raise ArnFp8Error("arnfp8_run_fmt", st)


def arnfp8_split_workspace_bytes(rows: int) -> int:
    """Bytes of the workspace ``arnfp8_run_split`` needs for ``rows`` rows (-1 if invalid)."""
    return int(library().arnfp8_split_workspace_bytes(int(rows)))


def arnfp8_split_parts(rows, cols) -> int:
    """Parts per row ``arnfp8_run_split`` picks automatically on the current
    device for ``rows`` x ``cols`` (-1 if the shape is not valid)."""
    return int(library().arnfp8_split_parts(int(rows), int(cols)))


def arnfp8_run_split(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                     weight_offset, scale_ub, rows=None, cols=None, P=None, workspace=None,
                     workspace_bytes=None, stream=None, opts=None) -> None:
    """The fused epilogue (e4m3fn) with each row split across several
    workgroups that trade their row statistics through ``workspace`` (a device
    tensor of at least ``arnfp8_split_workspace_bytes(rows)`` bytes, zeroed
    before its first use and then reused as is).  ``opts``: a ``SplitOpts``,
    a dict of its fields, or None.  The residual cannot be updated in place."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    if isinstance(opts, dict):
        opts = SplitOpts(**opts)
    opt = ctypes.byref(opts) if opts is not None else None
    n = rows * cols
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if workspace is not None and not isinstance(workspace, int) else 0)
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(out_fp8, _FP8, "out_fp8", n),
            _ptr(scales, _F32, "scales", 4 * rows), _ptr(gamma, _BF16, "gamma", 2 * cols))
    ws = _ptr(workspace, None, "workspace", None)
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               out_fp8=out_fp8, scales=scales, gamma=gamma, workspace=workspace)
    st = library().arnfp8_run_split(*ptrs, float(eps), float(weight_offset), float(scale_ub),
                                    rows, cols, P, ws, int(workspace_bytes), _stream(stream), opt)
    if st != 0:
        raise ArnFp8Error("arnfp8_run_split", st)


def arnfp8_run_split_noalloc(inputs, residual_in, residual_out, out_fp8, scales, gamma, eps,
                             weight_offset, scale_ub, rows=None, cols=None, P=None, stream=None,
                             opts=None) -> None:
    """``arnfp8_run_split`` with the library's own per-device workspace (at
    most ``NOALLOC_MAX_ROWS`` rows): allocates nothing.  Calls that may run at
    the same time on one device race (they share that workspace)."""
    rows, cols, P = _shape(inputs, rows, cols, P)
    if isinstance(opts, dict):
        opts = SplitOpts(**opts)
    opt = ctypes.byref(opts) if opts is not None else None
    n = rows * cols
    ptrs = (_ptr_array(inputs, 2 * n), _ptr(residual_in, _BF16, "residual_in", 2 * n),
            _ptr(residual_out, _BF16, "residual_out", 2 * n), _ptr(out_fp8, _FP8, "out_fp8", n),
            _ptr(scales, _F32, "scales", 4 * rows), _ptr(gamma, _BF16, "gamma", 2 * cols))
    _on_device(inputs=inputs, residual_in=residual_in, residual_out=residual_out,
               out_fp8=out_fp8, scales=scales, gamma=gamma)
    st = library().arnfp8_run_split_noalloc(*ptrs, float(eps), float(weight_offset),
                                            float(scale_ub), rows, cols, P, _stream(stream), opt)
    if st != 0:
        raise ArnFp8Error("arnfp8_run_split_noalloc", st)


def arnfp8_convert_f32(inp, out, fmt, n=None, stream=None) -> None:
    """The kernels' conversion step alone: fp32 ``inp`` -> ``out`` in format
    ``fmt`` (FMT_E4M3FN, FMT_E5M2: clamped; CVT_BF16), round to nearest even."""
    n = int(inp.numel()) if n is None else int(n)
    out_kinds = ("bfloat16", "int16", "uint16") if int(fmt) == CVT_BF16 else _FP8
    out_bytes = n * (2 if int(fmt) == CVT_BF16 else 1)
    ptrs = (_ptr(inp, _F32, "inp", 4 * n), _ptr(out, out_kinds, "out", out_bytes))
    _on_device(inp=inp, out=out)
    st = library().arnfp8_convert_f32(*ptrs, n, int(fmt), _stream(stream))
    if st != 0:
        raise ArnFp8Error("arnfp8_convert_f32", st)
