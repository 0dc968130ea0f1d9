"""Seeded synthetic inputs, shared by the GPU path, the tests and the benchmark.

This module holds none of the GEMM's arithmetic: it draws seeded random values, rounds them once
to an operand type, and lays them out with given element strides.  Everything that needs the
same input (the GPU library and the CPU oracle) receives the bits produced here.

Recipe (the pages measure on no dataset; every input is synthetic):
* values are drawn in float64 from numpy's PCG64 generator seeded with the given seed, in
  logical row-major order, so the same seed gives the same logical matrix in any storage order;
* they are rounded once from float64 to the operand type, to nearest with ties to even (float8 is
  OCP e4m3 "fn", saturating at +-448);
* storage is a flat array; element (r, c) sits at r * strides[0] + c * strides[1].
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

STORAGE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "e4m3": torch.float8_e4m3fn}
_TORCH_BITS = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def draw(seed: int, count: int, dist: str = "normal", *, std: float = 1.0, lo: float = -1.0,
         hi: float = 1.0) -> np.ndarray:
    """`count` float64 values: "normal" N(0, std^2), "uniform" U[lo, hi], or "dyadic" (multiples
    of 1/4 in [-1, 1], exactly representable in every operand type)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "normal":
        return rng.standard_normal(count) * std
    if dist == "uniform":
        return rng.uniform(lo, hi, count)
    if dist == "dyadic":
        return rng.integers(-4, 5, count).astype(np.float64) / 4.0
    raise ValueError(f"unknown distribution {dist!r}")


# (stored mantissa bits, smallest normal exponent, largest finite value) of the narrow types
_FORMAT = {"bf16": (7, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127), "e4m3": (3, -6, 448.0)}


def quantize(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to `dtype`, to nearest with ties to even; returns the stored
    bits.  f32 and f16 use numpy's direct conversions from double.  bf16 and e4m3 round at the
    value's quantum 2^(max(e, emin) - mbits) (e its binary exponent) with numpy's rint, which ties
    to even; the result is then exact in float32 and in the type, so the final casts are exact.
    bf16 overflows to infinity; e4m3 ("fn", no infinities) saturates to +-448."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    if dtype == "f32":
        with np.errstate(over="ignore"):           # beyond the float32 range: infinity
            return v.astype(np.float32).view(np.uint32).copy()
    if dtype == "f16":
        with np.errstate(over="ignore"):           # beyond 65504: infinity, as IEEE rounding gives
            return v.astype(np.float16).view(np.uint16).copy()
    mbits, emin, vmax = _FORMAT[dtype]
    with np.errstate(over="ignore", invalid="ignore"):
        _, ex = np.frexp(v)                        # v = f * 2^ex, 0.5 <= |f| < 1
        e = np.maximum(ex - 1, emin)
        q = np.ldexp(1.0, e - mbits)               # the quantum at v's exponent
        r = np.rint(v / q) * q                     # exact scalings; rint ties to even
        if dtype == "bf16":
            r = np.where(np.abs(r) > vmax, np.copysign(np.inf, v), r)
        else:
            r = np.clip(r, -vmax, vmax)
        r = np.where(np.isnan(v), np.nan, r)
    t = torch.from_numpy(r.astype(np.float32))     # exact: r has at most mbits + 1 bits
    bits = t.to(_TORCH[dtype]).view(_TORCH_BITS[dtype]).numpy()
    return bits.view(STORAGE[dtype]).copy()


@dataclasses.dataclass
class HostMatrix:
    storage: np.ndarray      # flat bits
    dtype: str
    shape: tuple             # (rows, cols)
    strides: tuple           # element strides (row, col)

    @property
    def nbytes(self) -> int:
        return self.storage.size * ESIZE[self.dtype]


def layout_strides(rows: int, cols: int, order: str, ld: int | None = None):
    """Strides of a row-major ("row", ld >= cols) or column-major ("col", ld >= rows) matrix."""
    if order == "row":
        ld = cols if ld is None else ld
        if ld < cols:
            raise ValueError("leading dimension below the row length")
        return (ld, 1), (rows - 1) * ld + cols if rows and cols else 0
    if order == "col":
        ld = rows if ld is None else ld
        if ld < rows:
            raise ValueError("leading dimension below the column length")
        return (1, ld), (cols - 1) * ld + rows if rows and cols else 0
    raise ValueError(f"unknown order {order!r}")


def place(bits_rowmajor: np.ndarray, rows: int, cols: int, dtype: str, order: str = "row",
          ld: int | None = None, fill: int = 0) -> HostMatrix:
    """Lay out logical row-major bits in the requested storage order."""
    strides, n = layout_strides(rows, cols, order, ld)
    if rows and cols and ld is None:
        # dense layouts: the logical bits themselves, or their transpose
        logical = np.ascontiguousarray(bits_rowmajor, dtype=STORAGE[dtype]).reshape(rows, cols)
        storage = logical.ravel() if order == "row" else np.ascontiguousarray(logical.T).ravel()
        return HostMatrix(storage.copy(), dtype, (rows, cols), strides)
    storage = np.full(max(n, 1) if rows and cols else 0, fill, dtype=STORAGE[dtype])
    if rows and cols:
        logical = bits_rowmajor.reshape(rows, cols)
        r = np.arange(rows, dtype=np.int64)[:, None]
        c = np.arange(cols, dtype=np.int64)[None, :]
        storage[(r * strides[0] + c * strides[1]).ravel()] = logical.ravel()
    return HostMatrix(storage, dtype, (rows, cols), strides)


def matrix(seed: int, rows: int, cols: int, dtype: str, dist: str = "normal", *,
           order: str = "row", ld: int | None = None, **params) -> HostMatrix:
    vals = draw(seed, rows * cols, dist, **params)
    return place(quantize(vals, dtype), rows, cols, dtype, order, ld)


def vector(seed: int, n: int, dtype: str, dist: str = "normal", **params) -> HostMatrix:
    bits = quantize(draw(seed, n, dist, **params), dtype)
    return HostMatrix(bits, dtype, (1, n), (n, 1))


def to_device(m: HostMatrix, device="cuda") -> torch.Tensor:
    """Upload the flat storage; the tensor is only a device buffer (its torch dtype is the
    storage integer type)."""
    t = torch.from_numpy(m.storage.view({1: np.uint8, 2: np.int16, 4: np.int32}[ESIZE[m.dtype]]))
    return t.to(device)
