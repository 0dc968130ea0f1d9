"""Split tail: when the tiles of a one-workgroup-per-CU kernel leave the last round of 256 at most
half full, the library splits each tile of that round along K and sums the slices in a second
kernel (the data-parallel plus split-K hybrid of Stream-K scheduling; the library takes Stream-K
itself for these shapes on kernels with a Stream-K form, so the tests ask for decomposition 1).  Checks the plan, exact
results on dyadic inputs (bit-identical to the unsplit run and to the oracle), and tolerance on
ordinary inputs for each operand type.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error, sample_indices

pytestmark = pytest.mark.gpu


RING = {"bf16": "bf16_ak_bk_256x256x64_w2x4_m16_ring", "f16": "f16_ak_bk_256x256x64_w2x4_m16_ring",
        "e4m3": "e4m3_ak_bk_256x256x128_w2x4_m32_ring"}


def plan(M, N, K, dtype="bf16", split_k=0):
    # the ring entry of the type, planned by the library; decomposition 1: no Stream-K, which
    # the plan otherwise takes for these last rounds on the rings that have a Stream-K form
    ring = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())].index(RING[dtype])
    g = H.Gemm(H.make_desc(M, N, K, dtype, (K, 1), (1, K), (N, 1), split_k=split_k,
                           decomposition=1, force_config=ring))
    return g.info, g.workspace_bytes


@pytest.mark.parametrize("shape,dtype,want", [
    # 17 x 17 = 289 tiles of 256 x 256: 33 in the second round; 64 k-tiles -> 7 slices of 10
    ((4352, 4352, 4096), "bf16", (33, 7)),
    ((6144, 6144, 4096), "bf16", (64, 4)),      # 576 tiles: 64 left, 256 / 64 = 4 slices
    ((8448, 8192, 8192), "bf16", (32, 8)),      # 33 x 32 = 1056 tiles: 32 left; 128 k-tiles
    ((4864, 4096, 4096), "f16", (48, 5)),       # 19 x 16 = 304 tiles, 64 k-tiles -> 5 of 13
    ((4352, 4352, 8192), "e4m3", (33, 7)),      # 128-element k-tiles: 64 -> 7 slices of 10
    ((4352, 4352, 2048), "bf16", (0, 1)),       # 32 k-tiles: too short to pay
    ((4352, 4352, 4096), "e4m3", (0, 1)),       # 32 k-tiles of 128
    ((8192, 8192, 8192), "bf16", (0, 1)),       # 1024 tiles: whole rounds
    ((5632, 5632, 4096), "bf16", (0, 1)),       # 484 tiles: last round 228 of 256, full enough
])
def test_plan(shape, dtype, want):
    info, ws = plan(*shape, dtype=dtype)
    assert "_ring" in info.name.decode()
    assert (info.tail_tiles, info.tail_split) == want
    if want[1] > 1:
        assert ws == want[0] * want[1] * 256 * 256 * 4
    forced, ws1 = plan(*shape, dtype=dtype, split_k=1)
    assert (forced.tail_tiles, forced.tail_split) == (0, 1) and ws1 == 0


def test_dyadic_exact_and_identical_to_unsplit():
    c = Case(4352, 4352, 4096, "bf16", "row", "col", dist="dyadic", alpha=2.0, beta=0.5,
             has_c=True, bias=True, seed=77, decomposition=1)
    p = Prepared(c)
    g, out = p.run()
    assert (g.info.tail_tiles, g.info.tail_split) == (33, 7)
    _, bits = p.decode_out(out)
    p1 = Prepared(dataclasses.replace(c, split_k=1))
    g1, out1 = p1.run()
    assert g1.info.tail_split == 1
    _, bits1 = p1.decode_out(out1)
    assert int((bits != bits1).sum()) == 0
    rows, cols = sample_indices(c.M, c.N, seed=3)
    want = oracle.encode_rne(OUT_T["bf16"], p.oracle_elems(rows, cols))
    assert int((bits[rows, cols] != want).sum()) == 0


@pytest.mark.parametrize("case", [
    Case(4352, 4352, 4096, "bf16", "row", "col", bias=True, act="gelu", seed=78, decomposition=1),
    Case(4864, 4096, 4096, "f16", "row", "col", has_c=True, beta=-0.5, alpha=0.75, seed=79,
         decomposition=1),
    Case(4352, 4352, 8192, "e4m3", "row", "col", std=1.0, scale_a=0.05, scale_b=0.05, seed=80,
         decomposition=1),
], ids=["bf16_gelu", "f16_c", "e4m3"])
def test_sampled_parity(case):
    p = Prepared(case)
    g, out = p.run()
    assert g.info.tail_split > 1
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    rows, cols = sample_indices(case.M, case.N, seed=4)
    err = error(case.dtype, got[rows, cols], p.oracle_elems(rows, cols))
    print(f"{case.dtype} {case.M}x{case.N}x{case.K}: {g.info.name.decode()} "
          f"tail {g.info.tail_tiles}x{g.info.tail_split} err={err:.3e}")
    assert err <= TOL[case.dtype], err
