"""Shared helpers for the GPU parity tests: build seeded inputs once, run the HIP library through
its C ABI, and compute the oracle on the same bits."""
from __future__ import annotations

import dataclasses
import os

import numpy as np
import torch

import oracle
from hierarchical_tiling_amd import htgemm as H
from hierarchical_tiling_amd import inputs

OUT_T = {"f32": "f32", "f16": "f16", "bf16": "bf16", "e4m3": "bf16"}
# host threads for the oracle: every core this process may use, at most 16 (the host threads that
# go with one GPU on an 8-GPU MI355X machine, whatever its core count)
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
# tolerances: fp32 relative Frobenius; 16-bit max-abs-relative; fp8 max-abs-relative
TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2, "e4m3": 3e-2}


@dataclasses.dataclass
class Case:
    M: int
    N: int
    K: int
    dtype: str
    a_order: str = "row"        # row-major A: unit stride along K
    b_order: str = "col"        # column-major B: unit stride along K
    dist: str = "normal"
    std: float | None = None    # None: 1/sqrt(K) for normal draws
    alpha: float = 1.0
    beta: float = 0.0
    has_c: bool = False
    bias: bool = False
    act: str = "none"
    scale_a: float = 1.0
    scale_b: float = 1.0
    a_ld: int | None = None
    b_ld: int | None = None
    c_ld: int | None = None
    d_ld: int | None = None
    d_order: str = "row"
    seed: int = 0
    force: int = -1
    a_offset: int = 0           # element offset of A's base pointer (misalignment tests)
    c_fill_nan: bool = False
    split_k: int = 0            # 0: the library decides; 1: never; >1: that many K slices
    row_scale: bool = False     # per-row fp32 scale vector (gemm_run_ex)
    col_scale: bool = False     # per-column fp32 scale vector (gemm_run_ex)
    scale_dist: str = "uniform"  # "uniform": U[0.25, 2] rows, U[-2, 2] columns; "pow2": 2^[-3..3]
    row_sumsq: bool = False     # also compute the row sums of squares of D (gemm_run_ex)
    col_sum: bool = False       # also compute the column sums of D (gemm_run_ex)
    decomposition: int = 0      # 0: the library decides; 1: no Stream-K; 2: Stream-K


def op(m):
    return oracle.Operand(m.storage, m.dtype, m.shape, m.strides)


class Prepared:
    def __init__(self, case: Case, device="cuda"):
        c = self.case = case
        s = c.seed * 10
        std = c.std if c.std is not None else (c.K ** -0.5 if c.K else 1.0)
        kw = dict(std=std) if c.dist == "normal" else {}
        self.A = inputs.matrix(s + 1, c.M, c.K, c.dtype, c.dist, order=c.a_order, ld=c.a_ld, **kw)
        self.B = inputs.matrix(s + 2, c.K, c.N, c.dtype, c.dist, order=c.b_order, ld=c.b_ld, **kw)
        ot = OUT_T[c.dtype]
        self.C = None
        if c.has_c:
            if c.c_fill_nan:
                nan_bits = oracle.encode_rne(ot, np.array([np.nan]))[0]
                self.C = inputs.place(np.full(c.M * c.N, nan_bits), c.M, c.N, ot, "row", c.c_ld)
            else:
                cdist = "dyadic" if c.dist == "dyadic" else "uniform"
                self.C = inputs.matrix(s + 3, c.M, c.N, ot, cdist, order="row", ld=c.c_ld)
        self.bias = None
        if c.bias:
            bdist = "dyadic" if c.dist == "dyadic" else "normal"
            self.bias = inputs.vector(s + 4, c.N, ot, bdist, **({"std": 0.1} if bdist == "normal" else {}))
        self.rs = self._scales(s + 5, c.M, 0.25) if c.row_scale else None
        self.cs = self._scales(s + 6, c.N, -2.0) if c.col_scale else None
        d_strides, n = inputs.layout_strides(c.M, c.N, c.d_order, c.d_ld)
        self.d_strides = d_strides
        self.d_len = max(n, 1)
        self.device = device
        self.dA = self._upload(self.A, c.a_offset)
        self.dB = inputs.to_device(self.B, device) if self.B.storage.size else torch.empty(1, device=device)
        self.dC = inputs.to_device(self.C, device) if self.C is not None else None
        self.dbias = inputs.to_device(self.bias, device) if self.bias is not None else None
        self.drs = torch.from_numpy(self.rs).to(device) if self.rs is not None else None
        self.dcs = torch.from_numpy(self.cs).to(device) if self.cs is not None else None

    def _scales(self, seed, n, lo):
        if self.case.scale_dist == "pow2":
            e = np.round(inputs.draw(seed, n, "uniform") * 3.0)
            return (2.0 ** e).astype(np.float32)
        u = inputs.draw(seed, n, "uniform")          # U[-1, 1]
        return (lo + (u + 1.0) * (2.0 - lo) / 2.0).astype(np.float32)

    def _upload(self, m, offset):
        if m.storage.size == 0:
            return (torch.empty(8, dtype=torch.uint8, device=self.device), 0)
        es = inputs.ESIZE[m.dtype]
        raw = np.zeros((m.storage.size + offset) * es, dtype=np.uint8)
        raw[offset * es:] = m.storage.view(np.uint8)
        t = torch.from_numpy(raw).to(self.device)
        return (t, 0)

    def desc(self):
        c = self.case
        return H.make_desc(c.M, c.N, c.K, c.dtype, self.A.strides, self.B.strides, self.d_strides,
                           c_strides=self.C.strides if self.C is not None else None,
                           has_bias=c.bias, act=c.act, force_config=c.force, split_k=c.split_k,
                           row_scale=c.row_scale, col_scale=c.col_scale, row_sumsq=c.row_sumsq,
                           col_sum=c.col_sum, decomposition=c.decomposition)

    def run(self, g: H.Gemm | None = None, out=None):
        c = self.case
        g = g or H.Gemm(self.desc())
        es_out = inputs.ESIZE[OUT_T[c.dtype]]
        if out is None:
            out = torch.zeros(self.d_len * es_out, dtype=torch.uint8, device=self.device)
        a_ptr = self.dA[0].data_ptr() + c.a_offset * inputs.ESIZE[c.dtype]
        ws_bytes = g.workspace_bytes
        # the workspace starts as NaN: every plane element a split run reads must be written first
        ws = torch.full((max(ws_bytes, 4) // 4,), float("nan"), dtype=torch.float32,
                        device=self.device) if ws_bytes else None
        self.rsq = (torch.full((max(c.M, 1),), float("nan"), dtype=torch.float32, device=self.device)
                    if c.row_sumsq else None)
        self.csum = (torch.full((max(c.N, 1),), float("nan"), dtype=torch.float32, device=self.device)
                     if c.col_sum else None)
        g.run(a_ptr, self.dB, self.dC, out, self.dbias, alpha=c.alpha, beta=c.beta,
              scale_a=c.scale_a, scale_b=c.scale_b, workspace=ws, row_scale=self.drs,
              col_scale=self.dcs, row_sumsq=self.rsq, col_sum=self.csum)
        torch.cuda.synchronize()
        return g, out

    def decode_out(self, out):
        c = self.case
        ot = OUT_T[c.dtype]
        bits = out.cpu().numpy().view(inputs.STORAGE[ot])
        vals = oracle.decode(ot, bits)
        r = np.arange(c.M)[:, None] * self.d_strides[0] + np.arange(c.N)[None, :] * self.d_strides[1]
        return vals[r], bits[r]

    def oracle_full(self):
        c = self.case
        return oracle.gemm(op(self.A), op(self.B), op(self.C) if self.C is not None else None,
                           op(self.bias) if self.bias is not None else None, alpha=c.alpha,
                           beta=c.beta, scale_a=c.scale_a, scale_b=c.scale_b, act=c.act,
                           row_scale=self.rs, col_scale=self.cs, threads=THREADS)

    def oracle_elems(self, rows, cols):
        c = self.case
        return oracle.gemm_elems(op(self.A), op(self.B), rows, cols,
                                 op(self.C) if self.C is not None else None,
                                 op(self.bias) if self.bias is not None else None, alpha=c.alpha,
                                 beta=c.beta, scale_a=c.scale_a, scale_b=c.scale_b, act=c.act,
                                 row_scale=self.rs, col_scale=self.cs, threads=THREADS)

    def oracle_rows(self, rows):
        """Oracle D of whole rows `rows` (len(rows) x N): the oracle's own GEMM on the gathered
        rows of A (and C, row_scale), so every operand element is decoded once."""
        c = self.case
        rows = np.asarray(rows, dtype=np.int64)
        A = _gather(self.A, rows, np.arange(c.K))
        C = _gather(self.C, rows, np.arange(c.N)) if self.C is not None else None
        return oracle.gemm(A, op(self.B), C, op(self.bias) if self.bias is not None else None,
                           alpha=c.alpha, beta=c.beta, scale_a=c.scale_a, scale_b=c.scale_b,
                           act=c.act, row_scale=self.rs[rows] if self.rs is not None else None,
                           col_scale=self.cs, threads=THREADS)

    def oracle_cols(self, cols):
        """Oracle D of whole columns `cols` (M x len(cols)), from the gathered columns of B (and
        C, bias, col_scale)."""
        c = self.case
        cols = np.asarray(cols, dtype=np.int64)
        B = _gather(self.B, np.arange(c.K), cols)
        C = _gather(self.C, np.arange(c.M), cols) if self.C is not None else None
        bias = (oracle.Operand(self.bias.storage[cols], self.bias.dtype, (1, cols.size), (cols.size, 1))
                if self.bias is not None else None)
        return oracle.gemm(op(self.A), B, C, bias, alpha=c.alpha, beta=c.beta,
                           scale_a=c.scale_a, scale_b=c.scale_b, act=c.act, row_scale=self.rs,
                           col_scale=self.cs[cols] if self.cs is not None else None,
                           threads=THREADS)

    def oracle_sample(self, got, seed=0, n_rows=64, n_cols=64, n_rand=4096):
        """The outputs of D the oracle computes at a size where the whole product would take too
        long on the host: n_rows whole rows and n_cols whole columns (the first and last of each
        among them) and n_rand random elements.  Returns (got values, oracle values, what was
        sampled), with `got` the decoded M x N device result."""
        c = self.case
        rng = np.random.default_rng(seed)
        rows = _pick(rng, c.M, n_rows)
        cols = _pick(rng, c.N, n_cols)
        r = rng.integers(0, c.M, n_rand)
        k = rng.integers(0, c.N, n_rand)
        want = np.concatenate([self.oracle_rows(rows).ravel(), self.oracle_cols(cols).ravel(),
                               self.oracle_elems(r, k)])
        have = np.concatenate([got[rows, :].ravel(), got[:, cols].ravel(), got[r, k]])
        what = (f"{rows.size} full rows, {cols.size} full columns and {n_rand} random outputs "
                f"({want.size} values, {100.0 * want.size / (c.M * c.N):.2f}% of D)")
        return have, want, what


def _pick(rng, n, count):
    """`count` distinct indices below n (all of them if n <= count), always with 0 and n - 1."""
    if n <= count:
        return np.arange(n, dtype=np.int64)
    mid = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid])).astype(np.int64)


def _gather(m, rows, cols):
    """Operand holding elements (rows[i], cols[j]) of host matrix m, row-major."""
    idx = rows[:, None] * m.strides[0] + cols[None, :] * m.strides[1]
    bits = m.storage[idx.ravel()] if idx.size else m.storage[:0]
    return oracle.Operand(bits, m.dtype, (rows.size, cols.size), (max(cols.size, 1), 1))


def error(dtype, got, want):
    """The error metric for `dtype`: relative Frobenius (fp32) or max-abs-relative."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if dtype == "f32":
        return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-300))


def sample_indices(M, N, seed=0, n_rand=4096, n_rows=2, n_cols=2):
    """Full rows and columns (first, last, random) plus random elements."""
    rng = np.random.default_rng(seed)
    rows_sel = sorted({0, M - 1, *rng.integers(0, M, n_rows).tolist()})
    cols_sel = sorted({0, N - 1, *rng.integers(0, N, n_cols).tolist()})
    r = [np.full(N, i) for i in rows_sel] + [np.arange(M) for _ in cols_sel] + [rng.integers(0, M, n_rand)]
    c = [np.arange(N) for _ in rows_sel] + [np.full(M, j) for j in cols_sel] + [rng.integers(0, N, n_rand)]
    return np.concatenate(r).astype(np.int64), np.concatenate(c).astype(np.int64)
