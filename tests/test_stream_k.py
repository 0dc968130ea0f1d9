"""Stream-K ("CUTLASS", Part IV Stage 2: a tile scheduler that splits K across blocks so every
processor gets an equal share of the work, then reduces the partial sums; its reference, Osama
et al. 2023): 256 persistent workgroups share the k-tile iterations of the last tiles equally,
pieces of a tile that several workgroups share are added in K order by a second kernel.  Checks
results against the oracle (edges, K tails, every operand type and B layout, many pieces per
tile, empty workgroups), bit-identity with the data-parallel run on dyadic inputs, and the plan
at a real shape."""
import dataclasses

import numpy as np
import pytest

import oracle
from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error, sample_indices

pytestmark = pytest.mark.gpu


def _index(name):
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())].index(name)


RING = {"bf16": "bf16_ak_bk_256x256x64_w2x4_m16_ring", "f16": "f16_ak_bk_256x256x64_w2x4_m16_ring",
        "bf16_bn": "bf16_ak_bn_256x256x64_w2x4_m16_ring", "f16_bn": "f16_ak_bn_256x256x64_w2x4_m16_ring"}

FULL_CASES = {
    # 4 x 6 = 24 tiles, 16 k-tiles: 384 iterations over 256 workgroups, 11 to 12 pieces a tile;
    # ragged M and N edges, C, bias, GELU
    "bf16_24_tiles": (Case(1000, 1300, 1000, "bf16", has_c=True, beta=0.5, bias=True, act="gelu",
                           seed=301), "bf16"),
    # row-major B kept as rows of k, a K tail (520 = 8 k-tiles + 8)
    "f16_rowB_ktail": (Case(1536, 1280, 520, "f16", b_order="row", bias=True, seed=302), "f16_bn"),
    # 12 tiles x 4 k-tiles: 48 iterations, 208 workgroups with none
    "f16_empty_wgs": (Case(1024, 768, 256, "f16", alpha=0.5, act="silu", seed=303), "f16"),
    "bf16_rowB": (Case(777, 1032, 640, "bf16", b_order="row", has_c=True, beta=-1.0, seed=304),
                  "bf16_bn"),
    "f16_c": (Case(513, 769, 2048, "f16", has_c=True, beta=0.25, alpha=2.0, seed=305), "f16"),
}


@pytest.mark.parametrize("name", list(FULL_CASES))
def test_stream_k_matches_oracle(name):
    case, ring = FULL_CASES[name]
    case = dataclasses.replace(case, force=_index(RING[ring]), decomposition=2)
    p = Prepared(case)
    g, out = p.run()
    info = g.info
    tiles = -(-case.M // 256) * -(-case.N // 256)
    assert info.sk_tiles == tiles and info.sk_wgs == 256
    assert g.workspace_bytes >= 2 * 256 * 256 * 256 * 4
    got, _ = p.decode_out(out)
    err = error(case.dtype, got, p.oracle_full())
    print(f"{name}: {info.name.decode()} sk_tiles {info.sk_tiles} err={err:.3e}")
    assert err <= TOL[case.dtype], err


def test_stream_k_after_whole_rounds_sampled():
    # 24 x 24 = 576 tiles: the first 512 run whole, the last 64 Stream-K
    c = Case(6144, 6144, 320, "bf16", bias=True, act="relu", seed=306,
             force=_index(RING["bf16"]), decomposition=2)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.sk_tiles == 64
    got, _ = p.decode_out(out)
    have, want, what = p.oracle_sample(got, seed=7)
    err = error("bf16", have, want)
    print(f"6144^2 x 320 Stream-K: {what} err={err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("shape", [(1280, 1536, 2048), (6144, 6144, 512)])
def test_dyadic_stream_k_bits_equal_data_parallel(shape):
    M, N, K = shape
    c = Case(M, N, K, "bf16", dist="dyadic", alpha=2.0, beta=0.5, has_c=True, bias=True,
             seed=307, force=_index(RING["bf16"]), decomposition=2)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.sk_tiles > 0
    _, bits = p.decode_out(out)
    p1 = Prepared(dataclasses.replace(c, decomposition=1, split_k=1))
    g1, out1 = p1.run()
    assert g1.info.sk_tiles == 0
    _, bits1 = p1.decode_out(out1)
    assert int((bits != bits1).sum()) == 0
    rows, cols = sample_indices(M, N, seed=5)
    want = oracle.encode_rne(OUT_T["bf16"], p.oracle_elems(rows, cols))
    assert int((bits[rows, cols] != want).sum()) == 0


def test_heuristic_stream_k_at_a_real_shape():
    # 17 x 17 = 289 tiles: a last round of 33, 64 k-tiles; GELU and bias; the ring entry, with
    # the library planning the decomposition
    c = Case(4352, 4352, 4096, "bf16", bias=True, act="gelu", seed=308, force=_index(RING["bf16"]))
    p = Prepared(c)
    g, out = p.run()
    info = g.info
    assert "_ring" in info.name.decode() and info.sk_tiles == 33 and info.tail_split == 1
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    have, want, what = p.oracle_sample(got, seed=9)
    err = error("bf16", have, want)
    print(f"4352^2 x 4096: {info.name.decode()} sk_tiles {info.sk_tiles}: {what} err={err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("case", [
    Case(4864, 4096, 4096, "f16", has_c=True, beta=-0.5, alpha=0.75, seed=309,
         force=_index(RING["f16"])),
    Case(4352, 4352, 4096, "f16", b_order="row", bias=True, act="gelu", seed=310,
         force=_index(RING["f16_bn"])),
    Case(4352, 4352, 4096, "bf16", b_order="row", bias=True, seed=311,
         force=_index(RING["bf16_bn"])),
], ids=["f16_c", "f16_rowB", "bf16_rowB"])
def test_heuristic_stream_k_other_types(case):
    p = Prepared(case)
    g, out = p.run()
    info = g.info
    assert info.sk_tiles > 0, info.name.decode()
    got, _ = p.decode_out(out)
    have, want, what = p.oracle_sample(got, seed=11)
    err = error(case.dtype, have, want)
    print(f"{case.dtype} {case.M}x{case.N}x{case.K}: {info.name.decode()} sk {info.sk_tiles}: "
          f"{what} err={err:.3e}")
    assert err <= TOL[case.dtype], err


def test_stream_k_with_scale_vectors():
    # both scale vectors and SiLU through the Stream-K pieces and the fix-up's epilogue
    c = Case(1000, 1300, 1000, "bf16", bias=True, act="silu", row_scale=True, col_scale=True,
             seed=312, force=_index(RING["bf16"]), decomposition=2)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.sk_tiles == 24
    got, _ = p.decode_out(out)
    err = error("bf16", got, p.oracle_full())
    print(f"Stream-K with scale vectors: err={err:.3e}")
    assert err <= TOL["bf16"], err


def test_stream_k_on_repacked_operands():
    # odd leading dimensions and K: aligned copies of A and B, then Stream-K over the last round
    # of 25 x 25 = 625 ring tiles (113 left) of 129 k-tiles (asked for: the kernel the library
    # prefers for the copies, the ping-pong kernel, has no Stream-K form)
    c = Case(6145, 6145, 8193, "f16", b_order="row", has_c=True, beta=0.5, seed=313,
             decomposition=2)
    p = Prepared(c)
    g, out = p.run()
    info = g.info
    assert info.repack == 1 and info.sk_tiles == 113, (info.repack, info.sk_tiles)
    got, _ = p.decode_out(out)
    have, want, what = p.oracle_sample(got, seed=13)
    err = error("f16", have, want)
    print(f"f16 6145^2 x 8193 repack + Stream-K: {what} err={err:.3e}")
    assert err <= TOL["f16"], err
