"""CPU oracle for the tiled dense GEMM and the shape:stride layout helper.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the GPU library
(``hierarchical_tiling_amd``) and imports nothing from it; both sides are handed the same seeded
inputs and nothing else.

* ``oracle.gemm`` / ``oracle.gemm_elems`` / ``oracle.decode`` / ``oracle.encode_rne`` wrap the
  plain-C triple loop in ``htoracle.c`` (double accumulation, exact decode of every input).
* ``oracle.row_sumsq`` / ``oracle.col_sum`` reduce the output as stored: each value rounded to
  the output type, then squared and summed along a row, or summed along a column, in double.
* ``oracle.layout`` holds the pointwise definitions of the layout algebra (evaluate, compose,
  coalesce, complement, divide, swizzle).
* ``oracle.tile`` holds the pages' tile-arithmetic and pipeline formulas.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, exact rational arithmetic or library routines (see each test).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "htoracle.c")
_LIB_PATH = os.path.join(_HERE, "libhtoracle.so")

# The oracle's own dtype and activation numbering (independent of the GPU library's header).
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ACTS = {"none": 0, "relu": 1, "gelu": 2, "silu": 3}
_STORAGE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}


def build(force: bool = True) -> str:
    """Compile htoracle.c with gcc into oracle/libhtoracle.so (host code only)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.oracle_decode.argtypes = [i32, vp, i64, vp]
        lib.oracle_encode_rne.argtypes = [i32, vp, i64, vp]
        common = [i64, i64, i64, i32, vp, i64, i64, i32, vp, i64, i64, i32, vp, i64, i64, i32, vp,
                  vp, vp, dbl, dbl, dbl, dbl, i32]
        lib.oracle_gemm.argtypes = common + [vp, i64, i64, i32]
        lib.oracle_gemm_elems.argtypes = common + [i64, vp, vp, vp, i32]
        lib.oracle_row_sumsq.argtypes = [i32, vp, i64, i64, i64, vp]
        lib.oracle_col_sum.argtypes = [i32, vp, i64, i64, i64, vp]
        for f in (lib.oracle_decode, lib.oracle_encode_rne, lib.oracle_gemm, lib.oracle_gemm_elems,
                  lib.oracle_row_sumsq, lib.oracle_col_sum):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    if n is not None:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode(dtype: str, bits) -> np.ndarray:
    """Exact decode of stored bits (numpy array of the storage type) to float64."""
    bits = np.ascontiguousarray(bits, dtype=_STORAGE[dtype])
    out = np.empty(bits.shape, dtype=np.float64)
    rc = _load().oracle_decode(DTYPES[dtype], _ptr(bits), bits.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out


def encode_rne(dtype: str, values) -> np.ndarray:
    """Round float64 values to `dtype` (nearest, ties to even); returns the stored bits."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=_STORAGE[dtype])
    rc = _load().oracle_encode_rne(DTYPES[dtype], _ptr(values), values.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_encode_rne failed ({rc})")
    return out


class Operand:
    """A matrix operand as storage bits plus element strides: element (r, c) is at
    storage[r * strides[0] + c * strides[1]]."""

    def __init__(self, storage, dtype: str, shape, strides):
        self.storage = np.ascontiguousarray(storage, dtype=_STORAGE[dtype])
        self.dtype = dtype
        self.shape = tuple(int(s) for s in shape)
        self.strides = tuple(int(s) for s in strides)


def _scale_vec(v, n, what):
    """A float32 scale vector of length n, or None."""
    if v is None:
        return None
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.shape != (n,):
        raise ValueError(f"{what} must have shape ({n},)")
    return v


def _common_args(M, N, K, A, B, C, bias, alpha, beta, scale_a, scale_b, act, row_scale=None,
                 col_scale=None):
    lib = _load()
    c_type = DTYPES[C.dtype] if C is not None else 0
    c_str = C.strides if C is not None else (0, 0)
    b_type = DTYPES[bias.dtype] if bias is not None else 0
    args = [M, N, K,
            DTYPES[A.dtype], _ptr(A.storage), A.strides[0], A.strides[1],
            DTYPES[B.dtype], _ptr(B.storage), B.strides[0], B.strides[1],
            c_type, _ptr(C.storage) if C is not None else None, c_str[0], c_str[1],
            b_type, _ptr(bias.storage) if bias is not None else None,
            _ptr(row_scale), _ptr(col_scale),
            float(alpha), float(beta), float(scale_a), float(scale_b), ACTS[act]]
    return lib, args


def gemm(A: Operand, B: Operand, C: Operand | None = None, bias: Operand | None = None, *,
         alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0, act="none", row_scale=None,
         col_scale=None, threads=None) -> np.ndarray:
    """The whole M x N result in float64 (unrounded), row-major.  row_scale (M) and col_scale (N)
    are float32 vectors that multiply row i / column j of alpha*sA*sB*(A@B)."""
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    rs, cs = _scale_vec(row_scale, M, "row_scale"), _scale_vec(col_scale, N, "col_scale")
    out = np.empty((M, N), dtype=np.float64)
    lib, args = _common_args(M, N, K, A, B, C, bias, alpha, beta, scale_a, scale_b, act, rs, cs)
    rc = lib.oracle_gemm(*args, _ptr(out), N, 1, _threads(threads))
    if rc:
        raise ValueError(f"oracle_gemm failed ({rc})")
    return out


def gemm_elems(A: Operand, B: Operand, rows, cols, C: Operand | None = None,
               bias: Operand | None = None, *, alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0,
               act="none", row_scale=None, col_scale=None, threads=None) -> np.ndarray:
    """Selected outputs D(rows[e], cols[e]) in float64."""
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    rs, cs = _scale_vec(row_scale, M, "row_scale"), _scale_vec(col_scale, N, "col_scale")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, dtype=np.float64)
    lib, args = _common_args(M, N, K, A, B, C, bias, alpha, beta, scale_a, scale_b, act, rs, cs)
    rc = lib.oracle_gemm_elems(*args, rows.size, _ptr(rows), _ptr(cols), _ptr(out),
                               _threads(threads))
    if rc:
        raise ValueError(f"oracle_gemm_elems failed ({rc})")
    return out


def _reduce(fn, D, out_type, n_out):
    D = np.ascontiguousarray(D, dtype=np.float64)
    if D.ndim != 2:
        raise ValueError("D must be a matrix")
    M, N = D.shape
    out = np.empty(n_out(M, N), dtype=np.float64)
    rc = fn(DTYPES[out_type], _ptr(D), M, N, N, _ptr(out))
    if rc:
        raise ValueError(f"{fn.__name__} failed ({rc})")
    return out


def row_sumsq(D, out_type: str) -> np.ndarray:
    """For each row i of the double result D: the sum over j of the square of D[i, j] rounded to
    `out_type` (the stored output), in double."""
    return _reduce(_load().oracle_row_sumsq, D, out_type, lambda M, N: M)


def col_sum(D, out_type: str) -> np.ndarray:
    """For each column j of the double result D: the sum over i of D[i, j] rounded to
    `out_type`, in double."""
    return _reduce(_load().oracle_col_sum, D, out_type, lambda M, N: N)
