"""gemm_run_noalloc (for callers that cannot allocate) against gemm_run_ex with a caller-owned
workspace: the same kernels on the same inputs, so the outputs agree bit for bit; two calls in a
row share the library's static scratch, the second with a smaller problem."""
import numpy as np
import pytest
import torch

from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error

pytestmark = pytest.mark.gpu


def _run_both(c):
    p = Prepared(c)
    g = H.Gemm(p.desc())
    need = g.workspace_bytes
    assert 0 < need <= H.GEMM_NOALLOC_SCRATCH_BYTES
    _, out_ex = p.run(g)                         # gemm_run(_ex) with a NaN-filled workspace
    rsq_ex = p.rsq.clone() if p.rsq is not None else None
    csum_ex = p.csum.clone() if p.csum is not None else None
    es = {"f32": 4, "f16": 2, "bf16": 2}[OUT_T[c.dtype]]
    out_na = torch.full_like(out_ex, 0x55)
    rsq_na = torch.full((max(c.M, 1),), float("nan"), device="cuda") if c.row_sumsq else None
    csum_na = torch.full((max(c.N, 1),), float("nan"), device="cuda") if c.col_sum else None
    a_ptr = p.dA[0].data_ptr() + c.a_offset * es
    H.gemm_run_noalloc(g.handle, a_ptr, p.dB.data_ptr(),
                       p.dC.data_ptr() if p.dC is not None else None, out_na.data_ptr(),
                       p.dbias.data_ptr() if p.dbias is not None else None,
                       p.drs.data_ptr() if p.drs is not None else None,
                       p.dcs.data_ptr() if p.dcs is not None else None, c.alpha, c.beta,
                       c.scale_a, c.scale_b, torch.cuda.current_stream().cuda_stream,
                       rsq_na.data_ptr() if rsq_na is not None else None,
                       csum_na.data_ptr() if csum_na is not None else None)
    torch.cuda.synchronize()
    assert torch.equal(out_ex, out_na)
    if rsq_ex is not None:
        assert torch.equal(rsq_ex, rsq_na)
    if csum_ex is not None:
        assert torch.equal(csum_ex, csum_na)
    got, _ = p.decode_out(out_na)
    assert error(c.dtype, got, p.oracle_full()) <= TOL[c.dtype]
    return g


def test_noalloc_split_k_two_calls_second_smaller():
    # split-K planes in the scratch: 4 x 512 x 384 fp32, then 3 x 200 x 136 on the same scratch
    g1 = _run_both(Case(512, 384, 64 * 40 + 8, "bf16", split_k=4, bias=True, act="gelu", seed=61))
    assert g1.info.split_k == 4
    g2 = _run_both(Case(200, 136, 64 * 9 + 40, "bf16", split_k=3, has_c=True, beta=-0.5, seed=62))
    assert g2.info.split_k == 3


def test_noalloc_reductions_two_calls_second_smaller():
    # the fused reductions' partials in the scratch
    _run_both(Case(300, 600, 320, "bf16", row_sumsq=True, col_sum=True, bias=True, seed=63))
    _run_both(Case(131, 97, 77, "f16", b_order="row", a_ld=81, b_ld=99, row_sumsq=True,
                   col_sum=True, has_c=True, beta=-1.0, seed=64))
