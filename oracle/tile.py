"""Tile arithmetic and pipeline formulas as the pages state them (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

* blog.ecitis.org, "CuTe DSL and CUDA Tile", section "A tile is a plan for reuse" (and its
  widget): an M x N output tile with reduction extent K performs 2MNK FLOPs; loading each input
  tile once and writing the output once moves b(MK + KN + MN) bytes for element width b; the
  widget's double-buffered plan keeps two copies of the A and B tiles in shared memory and asks
  whether they fit the budget.
* Same page, "Pipelining hides a wait only when another resource can work": n tiles with load
  time L and compute time C take n(L + C) serially and L + C + (n - 1) max(L, C) pipelined.
* "CUTLASS" (stanleyjacob.dev), Part V "the arithmetic-intensity story": per K-step a block
  reads Mt + Nt elements and does 2 Mt Nt FLOPs, so a square tile of side T has intensity T / b.
* "A10 - CuTe, CUTLASS & CuTile", section 5 "Performance Analysis": a square N^3 GEMM with fp16
  inputs and fp32 output moves 8 N^2 bytes, so its intensity is N / 4.
"""
from __future__ import annotations

from fractions import Fraction


def tile_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k


def tile_bytes(m: int, n: int, k: int, b: int) -> int:
    return b * (m * k + k * n + m * n)


def tile_intensity(m: int, n: int, k: int, b: int) -> Fraction:
    return Fraction(tile_flops(m, n, k), tile_bytes(m, n, k, b))


def double_buffer_bytes(m: int, n: int, k: int, b: int) -> int:
    """Two stages of the A tile (m x k) and the B tile (k x n)."""
    return 2 * b * (m * k + k * n)


def buffers_fit(m: int, n: int, k: int, b: int, budget_kib: int) -> bool:
    return double_buffer_bytes(m, n, k, b) <= budget_kib * 1024


def kstep_intensity(mt: int, nt: int, b: int) -> Fraction:
    return Fraction(2 * mt * nt, (mt + nt) * b)


def square_gemm_intensity_f16_in_f32_out(n: int) -> Fraction:
    flops = 2 * n ** 3
    moved = 2 * (n * n * 2) + n * n * 4
    return Fraction(flops, moved)


def pipeline_serial(n: int, load, compute):
    return n * (load + compute)


def pipeline_overlapped(n: int, load, compute):
    return load + compute + (n - 1) * max(load, compute)
