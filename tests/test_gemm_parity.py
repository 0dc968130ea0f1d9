"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the same seeded bits.

Tolerances: fp32 relative Frobenius <= 1e-5; bf16/fp16 max-abs-relative
<= 1e-2; fp8 <= 3e-2 (max-abs-relative = max|D - O| / max|O|, with O the unrounded double
oracle).  Dyadic inputs (multiples of 1/4, exact in every operand type) make every fp32 partial
sum exact, so there the rounded result must match the oracle bit for bit in any summation order.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error, sample_indices

pytestmark = pytest.mark.gpu


def table():
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]


def case_for_entry(i, name):
    dtype = name.split("_")[0]
    a_order = "row" if "_ak_" in name else "col"
    b_order = "col" if "_bk_" in name else "row"
    vec = name.endswith("_vec") or "_dma" in name or "_ring" in name or ("_pp" in name)
    # several tiles and a ragged tail in M and N; K spans several k-tiles with a tail
    if "_skinny" in name:
        # M below one 16-row atom, a ragged last column block, a K tail inside the last k-step,
        # and fewer k-steps than waves (some waves own no K)
        M, N, K = 13, 328, 272 if dtype == "e4m3" else 208
    elif vec:
        M, N, K = 264, 328, 272 if dtype == "e4m3" else 208  # odd k-tile counts, K tails
    else:
        M, N, K = 301, 257, 203
    variant = i % 4
    return Case(M=M, N=N, K=K, dtype=dtype, a_order=a_order, b_order=b_order, seed=i,
                force=i, has_c=variant in (1, 3), beta=(-1.25 if variant in (1, 3) else 0.0),
                alpha=0.75 if variant != 2 else 1.0, bias=variant >= 2,
                act=["none", "none", "gelu", "relu"][variant],
                scale_a=0.5 if dtype == "e4m3" else 1.0, scale_b=0.25 if dtype == "e4m3" else 1.0,
                dist="normal" if dtype != "f32" else "uniform")


@pytest.mark.parametrize("idx", range(len(table())) if os.path.exists(H.LIB_PATH) else [],
                         ids=lambda i: table()[i])
def test_every_table_entry_matches_oracle(idx):
    name = table()[idx]
    c = case_for_entry(idx, name)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.config == idx
    got, _ = p.decode_out(out)
    want = p.oracle_full()
    err = error(c.dtype, got, want)
    print(f"{name}: {c.M}x{c.N}x{c.K} err={err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[c.dtype], (name, err)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
@pytest.mark.parametrize("layout", ["row-col", "row-row", "col-col", "col-row"])
def test_dyadic_inputs_are_bit_exact(dtype, layout):
    a_order, b_order = layout.split("-")
    c = Case(M=200, N=136, K=320, dtype=dtype, a_order=a_order, b_order=b_order, dist="dyadic",
             alpha=2.0, beta=0.5, has_c=True, bias=True, seed=7,
             scale_a=0.5 if dtype == "e4m3" else 1.0, scale_b=2.0 if dtype == "e4m3" else 1.0)
    p = Prepared(c)
    _, out = p.run()
    _, bits = p.decode_out(out)
    want = oracle.encode_rne(OUT_T[dtype], p.oracle_full())
    mism = int((bits != want).sum())
    assert mism == 0, f"{mism} of {bits.size} outputs differ"


# ---- the benchmark workloads at their full sizes ----------------------------------------------
FULL = {
    "fp32_256": Case(256, 256, 256, "f32", "row", "row", dist="uniform", alpha=1.5, beta=0.5,
                     has_c=True, seed=1000),
    "bf16_4096": Case(4096, 4096, 4096, "bf16", "row", "col", seed=2000),
    "fp16_ragged": Case(4099, 3071, 2053, "f16", "row", "row", dist="uniform", alpha=0.75,
                        beta=-1.25, has_c=True, seed=3000),
    "bf16_8192_gelu": Case(8192, 8192, 8192, "bf16", "row", "col", bias=True, act="gelu",
                           seed=4000),
    # the headline product with row-major B (N-contiguous), its second layout row
    "bf16_8192_gelu_bn": Case(8192, 8192, 8192, "bf16", "row", "row", bias=True, act="gelu",
                              seed=4200),
    "e4m3_skinny": Case(16, 16384, 8192, "e4m3", "row", "col", std=1.0, scale_a=0.05,
                        scale_b=0.05, seed=5000),
    "e4m3_8192": Case(8192, 8192, 8192, "e4m3", "row", "col", std=1.0, scale_a=0.05,
                      scale_b=0.05, seed=5100),
}


def _full_or_sample(p, got, seed):
    """(device values, oracle values, description): all of D when the oracle finishes it in a
    few seconds, else 64 full rows, 64 full columns and 4096 random outputs."""
    c = p.case
    if c.M * c.N * c.K <= 256 ** 3 or c.M <= 16:
        return got.ravel(), p.oracle_full().ravel(), f"all {c.M * c.N} outputs"
    return p.oracle_sample(got, seed=seed)


@pytest.mark.parametrize("name", list(FULL))
def test_benchmark_workloads(name):
    c = FULL[name]
    p = Prepared(c)
    g, out = p.run()
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    have, want, what = _full_or_sample(p, got, seed=1)
    err = error(c.dtype, have, want)
    print(f"{name}: {g.info.name.decode()} err={err:.3e} on {what}")
    assert err <= TOL[c.dtype], err


# Dyadic inputs at every benchmark shape, with each shape's alpha/beta, C and bias but no
# activation and power-of-two fp8 scales: every fp32 partial sum is exact (|sum| <= K in steps
# of 1/16, K*16 < 2^24), so whatever kernel the library picks must round to the oracle's bits
# ("A10 - CuTe, CUTLASS & CuTile", section 6 Pitfall 5: exactly representable inputs make a
# tight comparison meaningful).
FULL_DYADIC = {
    "fp32_256": dict(alpha=1.5, beta=0.5, has_c=True),
    "bf16_4096": dict(),
    "fp16_ragged": dict(alpha=0.75, beta=-1.25, has_c=True),
    "bf16_8192_gelu": dict(bias=True),
    "bf16_8192_gelu_bn": dict(bias=True),
    "e4m3_skinny": dict(scale_a=0.5, scale_b=0.25),
    "e4m3_8192": dict(scale_a=0.5, scale_b=0.25),
}


@pytest.mark.parametrize("name", list(FULL_DYADIC))
def test_benchmark_shapes_dyadic_bit_exact(name):
    import dataclasses
    base = FULL[name]
    c = dataclasses.replace(base, dist="dyadic", std=None, act="none", seed=base.seed + 7,
                            **FULL_DYADIC[name])
    p = Prepared(c)
    g, out = p.run()
    got, bits = p.decode_out(out)
    have, want, what = _full_or_sample(p, got, seed=5)
    ot = OUT_T[c.dtype]
    want_r = oracle.decode(ot, oracle.encode_rne(ot, want))
    mism = int((have != want_r).sum())
    print(f"{name} dyadic: {g.info.name.decode()} mismatches {mism} on {what}")
    assert mism == 0, f"{mism} of {have.size} outputs differ ({g.info.name.decode()})"


# ---- edge cases ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 300, 17), (300, 1, 9), (7, 9, 1), (33, 65, 0)])
def test_tiny_and_degenerate_shapes(shape):
    M, N, K = shape
    c = Case(M, N, K, "bf16", has_c=True, beta=0.5, bias=True, alpha=1.5, seed=11)
    p = Prepared(c)
    _, out = p.run()
    got, _ = p.decode_out(out)
    assert error("bf16", got, p.oracle_full()) <= TOL["bf16"]


def test_beta_zero_ignores_nan_c():
    c = Case(130, 140, 96, "f16", has_c=True, beta=0.0, c_fill_nan=True, seed=12)
    p = Prepared(c)
    _, out = p.run()
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    assert error("f16", got, p.oracle_full()) <= TOL["f16"]


def test_misaligned_pointer_uses_fallback_path_with_same_result():
    # A's base 2 bytes off 16: the library takes its element-aligned fallback entry, whose
    # result is within tolerance of the oracle
    # (no split along K in any of the runs, so that all of them sum in the same order)
    base = Case(264, 264, 128, "bf16", seed=13, split_k=1)
    p0 = Prepared(base)
    g0, out0 = p0.run()
    vec_name = g0.info.name.decode()
    assert vec_name.endswith("_vec")
    shifted = Case(264, 264, 128, "bf16", seed=13, a_offset=1, split_k=1)
    p1 = Prepared(shifted)
    _, out1 = p1.run()
    assert error("bf16", p1.decode_out(out1)[0], p1.oracle_full()) <= TOL["bf16"]
    # the same tile and atom with the realigning and the element-wise loaders reads the
    # misaligned A into the same LDS tiles as the 16-byte loaders read the aligned one, so the
    # three results agree bit for bit
    names = table()
    for kind in ("realign", "narrow"):
        p2 = Prepared(Case(264, 264, 128, "bf16", seed=13, a_offset=1, split_k=1,
                           force=names.index(vec_name.replace("_vec", "_" + kind))))
        g2, out2 = p2.run()
        assert g2.info.name.decode().endswith(kind)
        assert torch.equal(out0, out2), kind


def test_column_major_output_and_padded_leading_dims():
    c = Case(190, 170, 150, "f32", "col", "row", dist="uniform", has_c=True, beta=-1.0,
             a_ld=200, b_ld=180, c_ld=171, d_ld=197, d_order="col", seed=14)
    p = Prepared(c)
    _, out = p.run()
    got, _ = p.decode_out(out)
    assert error("f32", got, p.oracle_full()) <= TOL["f32"]


def test_in_place_d_equals_c():
    c = Case(256, 192, 128, "bf16", has_c=True, beta=1.0, alpha=-0.5, seed=15)
    p = Prepared(c)
    want = p.oracle_full()
    g = H.Gemm(p.desc())
    a_ptr = p.dA[0].data_ptr()
    g.run(a_ptr, p.dB, p.dC, p.dC, None, alpha=c.alpha, beta=c.beta)
    torch.cuda.synchronize()
    got, _ = p.decode_out(p.dC.view(torch.uint8))
    assert error("bf16", got, want) <= TOL["bf16"]


@pytest.mark.parametrize("force,dtype", [("bf16_ak_bk_256x256x64_w2x4_m16_ring", "bf16"),
                                         ("f16_ak_bk_64x64x64_w2x2_m16_vec", "f16"),
                                         ("f32_ak_bk_64x64x32_w2x2_m16_vec", "f32")])
def test_c_and_d_bases_off_16_bytes(force, dtype):
    # C and D start 3 and 1 elements past a 16-byte boundary with padded leading dimensions that
    # keep every row off the grid as well: C is staged and D stored in D's own 16-byte grid
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    M, N, K = 300, 520, 256
    c = Case(M, N, K, dtype, has_c=True, beta=-0.75, alpha=1.25, bias=True, c_ld=N + 5,
             dist="uniform" if dtype == "f32" else "normal", seed=17, force=names.index(force))
    p = Prepared(c)
    want = p.oracle_full()
    ot = OUT_T[dtype]
    es = {"f32": 4, "f16": 2, "bf16": 2}[ot]
    d_ld = N + 3
    c_host = p.C.storage
    c_buf = torch.zeros((c_host.size + 8) * es, dtype=torch.uint8, device="cuda")
    c_buf[3 * es:3 * es + c_host.size * es] = torch.from_numpy(c_host.view(np.uint8)).to("cuda")
    sentinel = oracle.encode_rne(ot, np.array([np.nan]))[0]
    d_host = np.full(M * d_ld + 16, sentinel, dtype=c_host.dtype)
    d_buf = torch.from_numpy(d_host.view(np.uint8)).to("cuda")
    desc = p.desc()
    desc.d_stride_m, desc.d_stride_n = d_ld, 1
    g = H.Gemm(desc)
    assert g.info.name.decode() == force
    g.run(p.dA[0].data_ptr(), p.dB, c_buf.data_ptr() + 3 * es, d_buf.data_ptr() + es, p.dbias,
          alpha=c.alpha, beta=c.beta)
    torch.cuda.synchronize()
    bits = d_buf.cpu().numpy().view(c_host.dtype)[1:]
    r = np.arange(M)[:, None] * d_ld + np.arange(N)[None, :]
    inside = np.zeros(bits.size, dtype=bool)
    inside[r.ravel()] = True
    assert (bits[~inside] == sentinel).all(), "a write outside D's rows"
    got = oracle.decode(ot, bits[r])
    err = error(dtype, got, want)
    print(f"{force}: err={err:.3e}")
    assert err <= TOL[dtype], err


def test_repeated_runs_are_bitwise_identical():
    c = Case(1024, 768, 512, "bf16", bias=True, act="gelu", seed=16)
    p = Prepared(c)
    g, out1 = p.run()
    _, out2 = p.run(g)
    assert torch.equal(out1, out2)


def test_fused_gelu_equals_gemm_then_gelu():
    base = dict(M=512, N=384, K=256, dtype="bf16", bias=True, seed=17)
    pf = Prepared(Case(act="gelu", **base))
    pu = Prepared(Case(act="none", **base))
    got_f, _ = pf.decode_out(pf.run()[1])
    # unfused: the GEMM output in double through exact GELU, vs the fused kernel's output
    from math import erf, sqrt
    unf = pu.oracle_full()
    gelu = np.vectorize(lambda x: 0.5 * x * (1.0 + erf(x / sqrt(2.0))))(unf)
    assert error("bf16", got_f, gelu) <= TOL["bf16"]


def test_error_does_not_grow_faster_than_sqrt_k():
    errs = []
    for K in (256, 1024, 4096):
        c = Case(128, 128, K, "bf16", std=1.0, seed=18)
        p = Prepared(c)
        got, _ = p.decode_out(p.run()[1])
        want = p.oracle_full()
        errs.append(np.abs(got - want).max() / np.sqrt(K))
    assert errs[2] <= 4 * errs[0] + 1e-12, errs


# ---- split-K ("CUTLASS", Part III: K split across workgroups, partial sums reduced after) ----

def _name_index(name):
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    return names.index(name)


SPLIT_CASES = {
    # tiled 16-byte kernel, K tail inside the last slice, C and GELU in the reduction epilogue
    "bf16_tiled_s3": dict(M=200, N=136, K=64 * 7 + 8, dtype="bf16", split_k=3, has_c=True,
                          beta=-0.5, bias=True, act="gelu", alpha=0.75),
    # split-ring kernel forced, ragged M/N tiles, K tail
    "bf16_ring_s4": dict(M=264, N=328, K=64 * 9 + 16, dtype="bf16", split_k=4, bias=True,
                         force="bf16_ak_bk_256x256x64_w2x4_m32_ring"),
    "bf16_ring16_s2": dict(M=300, N=264, K=64 * 5 + 40, dtype="bf16", split_k=2, act="gelu",
                           force="bf16_ak_bk_256x256x64_w2x4_m16_ring"),
    "bf16_ring1_s3": dict(M=300, N=264, K=64 * 7 + 8, dtype="bf16", split_k=3, bias=True,
                          force="bf16_ak_bk_256x256x64_w2x4_m16_ring1"),
    "e4m3_ring_s3": dict(M=264, N=328, K=128 * 5 + 32, dtype="e4m3", split_k=3,
                         scale_a=0.5, scale_b=0.25, force="e4m3_ak_bk_256x256x128_w2x4_m32_ring"),
    # element-wise loaders (column-major A, row-major B, odd leading dims)
    "f16_narrow_s2": dict(M=99, N=70, K=203, dtype="f16", a_order="col", b_order="row", split_k=2,
                          has_c=True, beta=1.25, act="relu"),
    "f32_s5": dict(M=130, N=96, K=32 * 10, dtype="f32", dist="uniform", split_k=5, has_c=True,
                   beta=0.5, alpha=1.5),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_k_matches_oracle(name):
    kw = dict(SPLIT_CASES[name])
    if isinstance(kw.get("force"), str):
        kw["force"] = _name_index(kw["force"])
    c = Case(seed=40 + list(SPLIT_CASES).index(name), **kw)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.split_k == c.split_k, (g.info.split_k, c.split_k)
    assert g.workspace_bytes == c.split_k * c.M * c.N * 4
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    err = error(c.dtype, got, p.oracle_full())
    print(f"{name}: {g.info.name.decode()} split {g.info.split_k} err={err:.3e}")
    assert err <= TOL[c.dtype], (name, err)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3", "f32"])
def test_split_k_dyadic_is_bit_exact(dtype):
    # exact fp32 partial sums: the split result equals the unsplit one and the oracle bit for bit
    c = Case(M=136, N=200, K=320 if dtype != "e4m3" else 640, dtype=dtype, dist="dyadic",
             alpha=2.0, beta=0.5, has_c=True, bias=True, seed=47, split_k=3,
             scale_a=0.5 if dtype == "e4m3" else 1.0, scale_b=2.0 if dtype == "e4m3" else 1.0)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.split_k == 3
    _, bits = p.decode_out(out)
    want = oracle.encode_rne(OUT_T[dtype], p.oracle_full())
    assert int((bits != want).sum()) == 0


def test_split_k_automatic_on_few_tiles_and_long_k():
    # 512 x 512 has 16 tiles of 128 x 128; K = 16384 (256 k-tiles) -> the library splits K
    c = Case(M=512, N=512, K=16384, dtype="bf16", seed=48, bias=True)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.split_k > 1
    got, _ = p.decode_out(out)
    rows, cols = sample_indices(c.M, c.N, seed=2, n_rand=2048)
    err = error("bf16", got[rows, cols], p.oracle_elems(rows, cols))
    print(f"auto split {g.info.split_k}: {g.info.name.decode()} err={err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("layout", ["row-col", "row-row", "col-col", "col-row"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_realigned_loads_equal_element_loads(dtype, layout):
    # odd leading dimensions and a base 2 bytes off a dword: the realigning 16-byte loader and the
    # element-wise loader feed the same tile kernel (unsplit, as the cost model may plan a split
    # for one loader and not the other), so the outputs agree bit for bit
    a_order, b_order = layout.split("-")
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    a = "ak" if a_order == "row" else "am"
    b = "bk" if b_order == "col" else "bn"
    outs = []
    for kind in ("realign", "narrow"):
        c = Case(M=259, N=197, K=301, dtype=dtype, a_order=a_order, b_order=b_order, seed=51,
                 a_ld=261 if a_order == "col" else 303, b_ld=199 if b_order == "row" else 301,
                 has_c=True, beta=0.5, bias=True, act="gelu", a_offset=1, split_k=1,
                 force=names.index(f"{dtype}_{a}_{b}_128x128x64_w2x2_m32_{kind}"))
        p = Prepared(c)
        g, out = p.run()
        assert g.info.name.decode().endswith(kind)
        outs.append(out)
        if kind == "realign":
            got, _ = p.decode_out(out)
            assert error(dtype, got, p.oracle_full()) <= TOL[dtype]
    assert torch.equal(outs[0], outs[1])
