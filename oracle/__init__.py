"""CPU oracle for the fused sum + residual + RMSNorm + FP8 quant epilogue.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``all_reduce_rmsnorm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``arnfp8_oracle.c`` (plain C, fp64 norm statistics);
this module only builds it with gcc and marshals numpy arrays through ctypes.
bf16 tensors are ``numpy.uint16`` bit patterns, fp8 tensors ``numpy.uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "arnfp8_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_arnfp8.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def build() -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_arnfp8.so``."""
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first only if it is not built."""
    global _lib
    if _lib is None:
        path = os.environ.get("ARNFP8_ORACLE_LIB")  # a mutant build, for the pin-strength test
        if path is None:
            path = LIB_PATH
            if not os.path.exists(path):
                build()
        L = ctypes.CDLL(path)
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        L.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f32_to_e4m3fn_sat.restype = ctypes.c_uint8
        L.oracle_f32_to_e4m3fn_sat.argtypes = [ctypes.c_float]
        L.oracle_e5m2_to_f64.restype = ctypes.c_double
        L.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f32_to_e5m2_sat.restype = ctypes.c_uint8
        L.oracle_f32_to_e5m2_sat.argtypes = [ctypes.c_float]
        L.oracle_sum_bf16.restype = ctypes.c_int
        L.oracle_sum_bf16.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _u16p,
                                      ctypes.c_int64, ctypes.c_int64]
        L.oracle_arnfp8.restype = ctypes.c_int
        L.oracle_arnfp8.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _u16p, _u16p,
                                    _u8p, _f32p, _u16p, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_int64, ctypes.c_int64]
        L.oracle_arnfp8_e5m2.restype = ctypes.c_int
        L.oracle_arnfp8_e5m2.argtypes = L.oracle_arnfp8.argtypes
        _f64p = ctypes.POINTER(ctypes.c_double)
        L.oracle_norm_rows.restype = ctypes.c_int
        L.oracle_norm_rows.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _u16p, _u16p, _u16p,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_int64,
                                       ctypes.c_int64, _f64p]
        L.oracle_mx_shared_exp.restype = ctypes.c_int
        L.oracle_mx_shared_exp.argtypes = [_f64p, ctypes.c_int]
        L.oracle_mx_quantize_block.restype = None
        L.oracle_mx_quantize_block.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, _u8p]
        L.oracle_arnfp8_mx.restype = ctypes.c_int
        L.oracle_arnfp8_mx.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int, _u16p, _u16p, _u8p,
                                       _u8p, _u16p, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int64, ctypes.c_int64]
        L.oracle_share_rows.restype = None
        L.oracle_share_rows.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_int64)]
        L.oracle_stage_bytes.restype = ctypes.c_int64
        L.oracle_stage_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        L.oracle_stage_share.restype = ctypes.c_int
        L.oracle_stage_share.argtypes = [_u8p, _f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, _u8p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctype)


def _slabs(inputs):
    arrs = [np.ascontiguousarray(x, dtype=np.uint16) for x in inputs]
    shape = arrs[0].shape
    for a in arrs:
        assert a.shape == shape, "all slabs must share one shape"
    ptrs = (_u16p * len(arrs))(*[a.ctypes.data_as(_u16p) for a in arrs])
    return arrs, ptrs, shape


def _rows_cols(shape):
    cols = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    return rows, cols


# -------------------------------------------------------------- codecs ----

def bf16_to_f32(b: int) -> float:
    return lib().oracle_bf16_to_f32(int(b))


def f32_to_bf16(f: float) -> int:
    return lib().oracle_f32_to_bf16(float(f))


def e4m3fn_to_f64(code: int) -> float:
    return lib().oracle_e4m3fn_to_f64(int(code))


def f32_to_e4m3fn_sat(v: float) -> int:
    return lib().oracle_f32_to_e4m3fn_sat(float(v))


def e5m2_to_f64(code: int) -> float:
    return lib().oracle_e5m2_to_f64(int(code))


def f32_to_e5m2_sat(v: float) -> int:
    return lib().oracle_f32_to_e5m2_sat(float(v))


# ------------------------------------------------------- the operation ----

def sum_bf16(inputs) -> np.ndarray:
    """Rank-order fp32 sum of the bf16 slabs, rounded once to bf16."""
    arrs, ptrs, shape = _slabs(inputs)
    rows, cols = _rows_cols(shape)
    out = np.empty(shape, dtype=np.uint16)
    st = lib().oracle_sum_bf16(ptrs, len(arrs), _ptr(out, _u16p), rows, cols)
    if st != 0:
        raise ValueError(f"oracle_sum_bf16 failed with status {st}")
    return out


def _fused(fn, inputs, gamma, eps, weight_offset, scale_ub, residual_in, want_residual_out):
    arrs, ptrs, shape = _slabs(inputs)
    rows, cols = _rows_cols(shape)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    assert gamma.shape == (cols,)
    res_in = None
    if residual_in is not None:
        res_in = np.ascontiguousarray(residual_in, dtype=np.uint16)
        assert res_in.shape == shape
    res_out = np.empty(shape, dtype=np.uint16) if want_residual_out else None
    out = np.empty(shape, dtype=np.uint8)
    scales = np.empty((rows,), dtype=np.float32)
    st = fn(ptrs, len(arrs), _ptr(res_in, _u16p), _ptr(res_out, _u16p), _ptr(out, _u8p),
            _ptr(scales, _f32p), _ptr(gamma, _u16p), float(eps), float(weight_offset),
            float(scale_ub), rows, cols)
    if st != 0:
        raise ValueError(f"oracle fused call failed with status {st}")
    return out, scales, res_out


def arnfp8_e5m2(inputs, gamma, eps, weight_offset, scale_ub, residual_in=None,
                want_residual_out=True):
    """The fused epilogue with e5m2 output (per-row scale over 57344)."""
    return _fused(lib().oracle_arnfp8_e5m2, inputs, gamma, eps, weight_offset, scale_ub,
                  residual_in, want_residual_out)


def norm_rows(inputs, gamma, eps, weight_offset, residual_in=None):
    """The normalised rows y = h * r * g in fp64 (steps up to the norm)."""
    arrs, ptrs, shape = _slabs(inputs)
    rows, cols = _rows_cols(shape)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    res_in = None if residual_in is None else np.ascontiguousarray(residual_in, dtype=np.uint16)
    y = np.empty((rows, cols), dtype=np.float64)
    st = lib().oracle_norm_rows(ptrs, len(arrs), _ptr(res_in, _u16p), _ptr(None, _u16p),
                                _ptr(gamma, _u16p), float(eps), float(weight_offset), rows, cols,
                                y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if st != 0:
        raise ValueError(f"oracle_norm_rows failed with status {st}")
    return y


def mx_shared_exp(block) -> int:
    v = np.ascontiguousarray(block, dtype=np.float64)
    return lib().oracle_mx_shared_exp(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), v.size)


def mx_quantize_block(block, shared_exp: int) -> np.ndarray:
    v = np.ascontiguousarray(block, dtype=np.float64)
    codes = np.empty(v.size, dtype=np.uint8)
    lib().oracle_mx_quantize_block(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), v.size,
                                   int(shared_exp), _ptr(codes, _u8p))
    return codes


def arnfp8_mx(inputs, gamma, eps, weight_offset, residual_in=None, want_residual_out=True):
    """The fused epilogue with MXFP8 output: (codes u8 [rows, cols], E8M0 block
    scales u8 [rows, cols / 32], residual_out u16 or None)."""
    arrs, ptrs, shape = _slabs(inputs)
    rows, cols = _rows_cols(shape)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    res_in = None if residual_in is None else np.ascontiguousarray(residual_in, dtype=np.uint16)
    res_out = np.empty(shape, dtype=np.uint16) if want_residual_out else None
    out = np.empty(shape, dtype=np.uint8)
    bs = np.empty((rows, cols // 32), dtype=np.uint8)
    st = lib().oracle_arnfp8_mx(ptrs, len(arrs), _ptr(res_in, _u16p), _ptr(res_out, _u16p),
                                _ptr(out, _u8p), _ptr(bs, _u8p), _ptr(gamma, _u16p), float(eps),
                                float(weight_offset), rows, cols)
    if st != 0:
        raise ValueError(f"oracle_arnfp8_mx failed with status {st}")
    return out, bs, res_out


def arnfp8(inputs, gamma, eps, weight_offset, scale_ub, residual_in=None,
           want_residual_out=True):
    """The fused epilogue.  Returns ``(out_fp8 u8, scales f32 [rows], residual_out u16 or None)``.

    ``residual_out`` holds the updated residual when ``residual_in`` is given,
    and the bf16 sum when it is not (if ``want_residual_out``).
    """
    arrs, ptrs, shape = _slabs(inputs)
    rows, cols = _rows_cols(shape)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    assert gamma.shape == (cols,)
    res_in = None
    if residual_in is not None:
        res_in = np.ascontiguousarray(residual_in, dtype=np.uint16)
        assert res_in.shape == shape
    res_out = np.empty(shape, dtype=np.uint16) if want_residual_out else None
    out = np.empty(shape, dtype=np.uint8)
    scales = np.empty((rows,), dtype=np.float32)
    st = lib().oracle_arnfp8(ptrs, len(arrs), _ptr(res_in, _u16p), _ptr(res_out, _u16p),
                             _ptr(out, _u8p), _ptr(scales, _f32p), _ptr(gamma, _u16p),
                             float(eps), float(weight_offset), float(scale_ub), rows, cols)
    if st != 0:
        raise ValueError(f"oracle_arnfp8 failed with status {st}")
    return out, scales, res_out


# ------------------------------------------------ two-stage row share ----

SIMD_WIDTH = 16  # bytes: the scales of a staging slot are padded to this


def share_rows(rows: int, ngpus: int, rank: int):
    """(first row, row count) of rank ``rank``'s share."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    lib().oracle_share_rows(int(rows), int(ngpus), int(rank), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def stage_bytes(rows: int, cols: int, ngpus: int, simd_width: int = SIMD_WIDTH) -> int:
    return lib().oracle_stage_bytes(int(rows), int(cols), int(ngpus), int(simd_width))


def stage_share(out_fp8, scales, ngpus: int, rank: int, simd_width: int = SIMD_WIDTH,
                fill: int = 0) -> np.ndarray:
    """Rank ``rank``'s staging slot built from a full fused output; bytes the
    share does not fill hold ``fill``."""
    out_fp8 = np.ascontiguousarray(out_fp8, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1)
    rows, cols = out_fp8.shape
    slot = np.full((stage_bytes(rows, cols, ngpus, simd_width),), fill, dtype=np.uint8)
    st = lib().oracle_stage_share(_ptr(out_fp8, _u8p), _ptr(scales, _f32p), rows, cols, ngpus,
                                  rank, simd_width, _ptr(slot, _u8p))
    if st != 0:
        raise ValueError(f"oracle_stage_share failed with status {st}")
    return slot
