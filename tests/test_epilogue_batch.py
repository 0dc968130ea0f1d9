"""GPU parity for the fused-epilogue extensions and the batch mode, through the C ABI.

* Per-row / per-column fp32 scale vectors and SiLU ("CUTLASS", Part IV Stage 5: an epilogue
  visitor tree fuses a per-channel dequantisation scale and an activation while the accumulator
  is in registers; "A10 - CuTe, CUTLASS & CuTile", drill answer 8).
* A batch of L problems of one shape in one call ("CUTLASS, CuTe, and CUDA Tile", "Assembling a
  CUTLASS kernel": the problem shape [M, N, K, L]).

Tolerances as in test_gemm_parity; dyadic inputs with power-of-two scales
must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_tiling_amd import htgemm as H
from hierarchical_tiling_amd import inputs
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error, op

pytestmark = pytest.mark.gpu


def _index(name):
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())].index(name)


EPI_CASES = {
    # split ring, 16x16 MFMA: both vectors, bias, SiLU, ragged M/N and a K tail
    "bf16_ring_scales_silu": dict(M=300, N=264, K=64 * 5 + 24, dtype="bf16", row_scale=True,
                                  col_scale=True, bias=True, act="silu",
                                  force="bf16_ak_bk_256x256x64_w2x4_m16_ring"),
    # library choice (tiled 16-byte kernel), column scale with C and GELU
    "bf16_colscale_c_gelu": dict(M=200, N=136, K=200, dtype="bf16", col_scale=True, has_c=True,
                                 beta=0.5, act="gelu"),
    # realigned loader (odd leading dims), row scale, C and SiLU
    "f16_realign_rowscale_silu": dict(M=131, N=97, K=77, dtype="f16", b_order="row", a_ld=81,
                                      b_ld=99, row_scale=True, has_c=True, beta=-1.0, act="silu"),
    # streaming skinny kernel with per-token and per-channel dequantisation scales
    "e4m3_skinny_scales": dict(M=16, N=1040, K=1024, dtype="e4m3", row_scale=True,
                               col_scale=True, scale_a=0.5, scale_b=0.25),
    "e4m3_ring_colscale_silu": dict(M=264, N=328, K=128 * 4 + 32, dtype="e4m3", col_scale=True,
                                    act="silu", force="e4m3_ak_bk_256x256x128_w2x4_m32_ring"),
    # split-K: the scales are applied in the reduction's epilogue
    "f32_split_scales_silu": dict(M=130, N=96, K=32 * 10, dtype="f32", dist="uniform", split_k=5,
                                  row_scale=True, col_scale=True, has_c=True, beta=0.5,
                                  alpha=1.5, act="silu"),
    "bf16_ring_split_scales": dict(M=264, N=328, K=64 * 9 + 16, dtype="bf16", split_k=3,
                                   row_scale=True, col_scale=True, bias=True, act="gelu",
                                   force="bf16_ak_bk_256x256x64_w2x4_m32_ring"),
}


@pytest.mark.parametrize("name", list(EPI_CASES))
def test_scale_vectors_and_silu_match_oracle(name):
    kw = dict(EPI_CASES[name])
    if isinstance(kw.get("force"), str):
        kw["force"] = _index(kw["force"])
    c = Case(seed=60 + list(EPI_CASES).index(name), **kw)
    p = Prepared(c)
    g, out = p.run()
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    err = error(c.dtype, got, p.oracle_full())
    print(f"{name}: {g.info.name.decode()} split {g.info.split_k} err={err:.3e}")
    assert err <= TOL[c.dtype], (name, err)


@pytest.mark.parametrize("dtype,force", [("bf16", "bf16_ak_bk_256x256x64_w2x4_m16_ring"),
                                         ("e4m3", "e4m3_ak_bk_256x256x128_w2x4_m32_ring"),
                                         ("f32", None), ("f16", None)])
def test_power_of_two_scales_are_bit_exact(dtype, force):
    # dyadic inputs and power-of-two scales keep every fp32 step exact: the rounded output must be
    # the rounded oracle bit for bit
    c = Case(M=264, N=200, K=256 if dtype != "e4m3" else 512, dtype=dtype, dist="dyadic",
             row_scale=True, col_scale=True, scale_dist="pow2", alpha=0.5, beta=2.0, has_c=True,
             bias=True, seed=71, force=_index(force) if force else -1)
    p = Prepared(c)
    g, out = p.run()
    _, bits = p.decode_out(out)
    want = oracle.encode_rne(OUT_T[dtype], p.oracle_full())
    assert int((bits != want).sum()) == 0, g.info.name.decode()


def test_fused_silu_equals_gemm_then_silu():
    base = dict(M=384, N=512, K=320, dtype="bf16", bias=True, seed=72, col_scale=True)
    pf = Prepared(Case(act="silu", **base))
    pu = Prepared(Case(act="none", **base))
    got_f, _ = pf.decode_out(pf.run()[1])
    unf = pu.oracle_full()
    silu = unf / (1.0 + np.exp(-unf))
    assert error("bf16", got_f, silu) <= TOL["bf16"]


def test_scale_vector_presence_must_match_the_handle():
    c = Case(M=64, N=64, K=64, dtype="bf16", row_scale=True, seed=73)
    p = Prepared(c)
    g = H.Gemm(p.desc())
    out = torch.zeros(64 * 64 * 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(H.GemmError) as e:   # gemm_run cannot pass the vector
        H.gemm_run(g.handle, p.dA[0].data_ptr(), p.dB.data_ptr(), None, out.data_ptr(), None,
                   1.0, 0.0)
    assert e.value.status == H.GEMM_ERR_INVALID_ARG
    with pytest.raises(H.GemmError) as e:   # gemm_run_ex without it
        H.gemm_run_ex(g.handle, p.dA[0].data_ptr(), p.dB.data_ptr(), None, out.data_ptr(), None,
                      None, None, 1.0, 0.0)
    assert e.value.status == H.GEMM_ERR_INVALID_ARG
    with pytest.raises(H.GemmError) as e:   # a column vector the handle does not have
        H.gemm_run_ex(g.handle, p.dA[0].data_ptr(), p.dB.data_ptr(), None, out.data_ptr(), None,
                      p.drs.data_ptr(), p.drs.data_ptr(), 1.0, 0.0)
    assert e.value.status == H.GEMM_ERR_INVALID_ARG
    with pytest.raises(H.GemmError) as e:   # misaligned vector
        H.gemm_run_ex(g.handle, p.dA[0].data_ptr(), p.dB.data_ptr(), None, out.data_ptr(), None,
                      p.drs.data_ptr() + 2, None, 1.0, 0.0)
    assert e.value.status == H.GEMM_ERR_MISALIGNED
    torch.cuda.synchronize()


# ---- batch (the L mode) ------------------------------------------------------------------------

def _stack(mats, pad_elems, align_elems):
    """Concatenate equal-size storages with one fixed stride between them."""
    n = mats[0].storage.size
    # pad > 0 keeps the odd stride (a problem base off the 16-byte grid); else round up
    stride = n + pad_elems if pad_elems else -(-n // align_elems) * align_elems
    flat = np.zeros(stride * len(mats), dtype=mats[0].storage.dtype)
    for i, m in enumerate(mats):
        flat[i * stride:i * stride + n] = m.storage
    return flat, stride


def _dev(flat):
    view = {1: np.uint8, 2: np.int16, 4: np.int32}[flat.dtype.itemsize]
    return torch.from_numpy(np.ascontiguousarray(flat).view(view)).to("cuda")


BATCH_CASES = {
    # split ring, distinct A/B per problem
    "bf16_ring_L3": dict(L=3, M=264, N=328, K=320, dtype="bf16", bias=True, act="gelu",
                         force="bf16_ak_bk_256x256x64_w2x4_m16_ring"),
    # a batch stride that is not a multiple of 16 bytes: the library must leave the 16-byte path
    "bf16_odd_stride_L2": dict(L=2, M=100, N=72, K=96, dtype="bf16", pad=1, has_c=True, beta=0.5),
    # skinny streaming kernel, B shared by every problem (stride 0), scale vectors
    "e4m3_skinny_sharedB_L4": dict(L=4, M=16, N=520, K=512, dtype="e4m3", shared_b=True,
                                   row_scale=True, col_scale=True, scale_a=0.5, scale_b=0.5),
    # fp32 with C, MN-major B
    "f32_C_L2": dict(L=2, M=70, N=90, K=50, dtype="f32", dist="uniform", b_order="row",
                     has_c=True, beta=-0.5, alpha=2.0),
    "f16_rowB_silu_L3": dict(L=3, M=96, N=128, K=64, dtype="f16", b_order="row", act="silu",
                             col_scale=True),
    # ping-pong kernel, K-major and row-major B
    "bf16_pp_L3": dict(L=3, M=264, N=328, K=320, dtype="bf16", bias=True, act="gelu",
                       force="bf16_ak_bk_256x256x64_w2x4_m16_pp"),
    "f16_pp_rowB_L2": dict(L=2, M=264, N=328, K=200, dtype="f16", b_order="row", has_c=True,
                           beta=-0.5, force="f16_ak_bn_256x256x64_w2x4_m16_pp"),
}


@pytest.mark.parametrize("name", list(BATCH_CASES))
def test_batched_problems_match_oracle_each(name):
    kw = dict(BATCH_CASES[name])
    L = kw.pop("L")
    pad = kw.pop("pad", 0)
    shared_b = kw.pop("shared_b", False)
    force = kw.pop("force", None)
    base_seed = 80 + list(BATCH_CASES).index(name) * 10
    preps = [Prepared(Case(seed=base_seed + l, **kw)) for l in range(L)]
    c0, p0 = preps[0].case, preps[0]
    ot = OUT_T[c0.dtype]
    align = 16 // inputs.ESIZE[c0.dtype]
    a_flat, sa = _stack([p.A for p in preps], pad, align)
    if shared_b:
        b_flat, sb = p0.B.storage, 0
    else:
        b_flat, sb = _stack([p.B for p in preps], pad, align)
    c_flat, sc = (_stack([p.C for p in preps], 0, 8) if c0.has_c else (None, 0))
    d_len = p0.d_len
    sd = -(-(d_len + 5) // 8) * 8       # a gap after every problem's D, checked below
    out_bits = oracle.encode_rne(ot, np.array([np.nan]))[0]
    d_host = np.full(sd * L, out_bits, dtype=inputs.STORAGE[ot])
    dA, dB, dD = _dev(a_flat), _dev(b_flat), _dev(d_host)
    dC = _dev(c_flat) if c_flat is not None else None
    desc = H.make_desc(c0.M, c0.N, c0.K, c0.dtype, p0.A.strides, p0.B.strides, p0.d_strides,
                       c_strides=p0.C.strides if p0.C is not None else None, has_bias=c0.bias,
                       act=c0.act, force_config=_index(force) if force else -1,
                       row_scale=c0.row_scale, col_scale=c0.col_scale, batch=L,
                       batch_strides=(sa, sb, sc, sd))
    g = H.Gemm(desc)
    info = g.info
    tiles = -(-c0.M // info.bm) * -(-c0.N // info.bn)
    assert info.grid == tiles * L and info.split_k == 1
    if pad:
        assert "_vec" not in info.name.decode() and "_ring" not in info.name.decode()
    g.run(dA, dB, dC, dD, p0.dbias, alpha=c0.alpha, beta=c0.beta, scale_a=c0.scale_a,
          scale_b=c0.scale_b, row_scale=p0.drs, col_scale=p0.dcs)
    torch.cuda.synchronize()
    d_all = dD.cpu().numpy().view(inputs.STORAGE[ot])
    r = np.arange(c0.M)[:, None] * p0.d_strides[0] + np.arange(c0.N)[None, :] * p0.d_strides[1]
    written = np.zeros(sd, dtype=bool)
    written[r.ravel()] = True
    for l, p in enumerate(preps):
        seg = d_all[l * sd:(l + 1) * sd]
        assert (seg[~written] == out_bits).all(), f"problem {l} wrote outside its D"
        got = oracle.decode(ot, seg)[r]
        B = p0.B if shared_b else p.B
        want = oracle.gemm(op(p.A), op(B), op(p.C) if p.C is not None else None,
                           op(p0.bias) if p0.bias is not None else None, alpha=c0.alpha,
                           beta=c0.beta, scale_a=c0.scale_a, scale_b=c0.scale_b, act=c0.act,
                           row_scale=p0.rs, col_scale=p0.cs)
        err = error(c0.dtype, got, want)
        print(f"{name}[{l}]: {info.name.decode()} err={err:.3e}")
        assert err <= TOL[c0.dtype], (name, l, err)


# ---- grouped GEMM with ragged M (mixture-of-experts) -----------------------------------------

GROUP_CASES = {
    # split ring: an empty group, a one-row group and groups spanning tile boundaries
    "bf16_ring_moe": dict(sizes=[300, 0, 1, 517, 211], N=264, K=320, dtype="bf16", bias=True,
                          act="silu", row_scale=True, col_scale=True,
                          force="bf16_ak_bk_256x256x64_w2x4_m16_ring"),
    # ping-pong kernel: the same group shapes
    "bf16_pp_moe": dict(sizes=[300, 0, 1, 517, 211], N=264, K=320, dtype="bf16", bias=True,
                        act="gelu", row_scale=True, force="bf16_ak_bk_256x256x64_w2x4_m16_pp"),
    "e4m3_pp_moe": dict(sizes=[260, 3, 0, 250], N=520, K=384, dtype="e4m3", scale_a=0.5,
                        scale_b=0.25, force="e4m3_ak_bk_256x256x128_w2x4_m16_pp"),
    "bf16_lib_moe_c": dict(sizes=[17, 128, 0, 95], N=200, K=128, dtype="bf16", has_c=True,
                           beta=0.5),
    # MN-major B per expert (tiled kernel), GELU
    "f16_rowB_moe": dict(sizes=[40, 77, 10], N=96, K=64, dtype="f16", b_order="row", act="gelu"),
    # 33 rows in all: the streaming skinny kernel must not be chosen for a grouped launch
    "e4m3_moe_small": dict(sizes=[3, 9, 0, 14, 2, 5], N=520, K=512, dtype="e4m3", scale_a=0.5,
                           scale_b=0.25),
    "f32_moe_c": dict(sizes=[33, 31], N=40, K=50, dtype="f32", dist="uniform", has_c=True,
                      beta=-1.0, alpha=2.0),
    # 3000 groups of 0..7 rows: several offsets per thread of the scan that builds the tile table
    "bf16_3000_groups": dict(sizes=[int(v) for v in np.random.default_rng(5).integers(0, 8, 3000)],
                             N=64, K=64, dtype="bf16", bias=True),
    # offsets out of range and decreasing: clamped into [0, M] and made non-decreasing, so the
    # groups are rows [0, 50), [50, 50), [50, 180), [180, 180), [180, 180); no row is left out
    "bf16_clamped_offsets": dict(raw_offsets=[-5, 50, 30, 200, 150, 400], M=180, N=72, K=64,
                                 dtype="bf16"),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_grouped_ragged_m_matches_oracle_per_group(name):
    kw = dict(GROUP_CASES[name])
    if "raw_offsets" in kw:
        offsets = np.array(kw.pop("raw_offsets"), dtype=np.int32)
        M = kw.pop("M")
        G = offsets.size - 1
    else:
        sizes = kw.pop("sizes")
        G, M = len(sizes), int(sum(sizes))
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    # the offsets as the library reads them: clamped into [0, M], made non-decreasing
    eff = np.minimum(np.maximum.accumulate(np.maximum(offsets, 0)), M)
    force = kw.pop("force", None)
    b_order = kw.pop("b_order", "col")
    seed = 200 + list(GROUP_CASES).index(name) * 10
    p = Prepared(Case(M=M, seed=seed, b_order=b_order, **kw))   # A, C, D, bias, scale vectors
    c = p.case
    std = c.K ** -0.5 if c.dist == "normal" else None
    bkw = dict(std=std) if std else {}
    Bs = [inputs.matrix(seed + 5 + e, c.K, c.N, c.dtype, c.dist, order=b_order, **bkw)
          for e in range(G)]
    b_flat, sb = _stack(Bs, 0, 16)
    ot = OUT_T[c.dtype]
    tail = 37                                                     # sentinel after D
    d_rows = M * p.d_strides[0]
    sentinel = oracle.encode_rne(ot, np.array([np.nan]))[0]
    d_host = np.full(d_rows + tail, sentinel, dtype=inputs.STORAGE[ot])
    dB, dD = _dev(b_flat), _dev(d_host)
    doff = torch.from_numpy(offsets).to("cuda")
    desc = H.make_desc(M, c.N, c.K, c.dtype, p.A.strides, Bs[0].strides, p.d_strides,
                       c_strides=p.C.strides if p.C is not None else None, has_bias=c.bias,
                       act=c.act, force_config=_index(force) if force else -1,
                       row_scale=c.row_scale, col_scale=c.col_scale, batch=G,
                       batch_strides=(0, sb, 0, 0), ragged_m=True)
    g = H.Gemm(desc)
    info = g.info
    assert b"skinny" not in info.name and info.split_k == 1
    assert info.grid == (-(-M // info.bm) + G) * -(-c.N // info.bn)
    a_ptr = p.dA[0].data_ptr()
    # the groups' tile table lives in the workspace, which starts as garbage
    assert g.workspace_bytes >= (G + 1) * 12
    ws = torch.full((g.workspace_bytes // 4,), -1, dtype=torch.int32, device="cuda")
    H.gemm_run_grouped(g.handle, a_ptr, dB.data_ptr(), p.dC.data_ptr() if p.dC is not None else None,
                       dD.data_ptr(), p.dbias.data_ptr() if p.dbias is not None else None,
                       p.drs.data_ptr() if p.drs is not None else None,
                       p.dcs.data_ptr() if p.dcs is not None else None, doff.data_ptr(),
                       c.alpha, c.beta, c.scale_a, c.scale_b,
                       torch.cuda.current_stream().cuda_stream, ws.data_ptr())
    torch.cuda.synchronize()
    d_all = dD.cpu().numpy().view(inputs.STORAGE[ot])
    assert (d_all[d_rows:] == sentinel).all(), "a group wrote past D"
    vals = oracle.decode(ot, d_all[:d_rows])
    ld_a, ld_d = p.A.strides[0], p.d_strides[0]
    covered = np.zeros(M, dtype=bool)
    for e in range(G):
        lo, hi = int(eff[e]), int(eff[e + 1])
        if hi == lo:
            continue
        covered[lo:hi] = True
        A_e = oracle.Operand(p.A.storage[lo * ld_a:], c.dtype, (hi - lo, c.K), p.A.strides)
        C_e = (oracle.Operand(p.C.storage[lo * p.C.strides[0]:], ot, (hi - lo, c.N), p.C.strides)
               if p.C is not None else None)
        want = oracle.gemm(A_e, op(Bs[e]), C_e, op(p.bias) if p.bias is not None else None,
                           alpha=c.alpha, beta=c.beta, scale_a=c.scale_a, scale_b=c.scale_b,
                           act=c.act, row_scale=p.rs[lo:hi] if p.rs is not None else None,
                           col_scale=p.cs, threads=1)
        r = np.arange(lo, hi)[:, None] * ld_d + np.arange(c.N)[None, :] * p.d_strides[1]
        got = vals[r]
        err = error(c.dtype, got, want)
        if G <= 16:
            print(f"{name}[{e}] rows {lo}:{hi}: {info.name.decode()} err={err:.3e}")
        assert err <= TOL[c.dtype], (name, e, lo, hi, err)
    # rows outside every group are not written
    rows_out = np.flatnonzero(~covered)
    if rows_out.size:
        r = rows_out[:, None] * ld_d + np.arange(c.N)[None, :] * p.d_strides[1]
        assert (d_all[r] == sentinel).all()


# ---- fused reductions: row sums of squares (the next layer's norm) and column sums ------------

RSQ_CASES = {
    "bf16_ring_gelu": dict(M=300, N=600, K=320, dtype="bf16", bias=True, act="gelu",
                           force="bf16_ak_bk_256x256x64_w2x4_m16_ring"),
    "f16_realign_c": dict(M=131, N=97, K=77, dtype="f16", b_order="row", a_ld=81, b_ld=99,
                          has_c=True, beta=-1.0),
    "e4m3_ring_scales": dict(M=264, N=328, K=256, dtype="e4m3", scale_a=0.5, scale_b=0.25,
                             col_scale=True, force="e4m3_ak_bk_256x256x128_w2x4_m32_ring"),
    "f32_uniform": dict(M=130, N=300, K=64, dtype="f32", dist="uniform"),
    "bf16_pp_gelu": dict(M=300, N=600, K=320, dtype="bf16", bias=True, act="gelu",
                         force="bf16_ak_bk_256x256x64_w2x4_m16_pp"),
    "e4m3_pp_scales": dict(M=264, N=328, K=256, dtype="e4m3", scale_a=0.5, scale_b=0.25,
                           col_scale=True, force="e4m3_ak_bk_256x256x128_w2x4_m16_pp"),
    # 16 rows would take the streaming skinny kernel, which has no row reduction
    "bf16_m16": dict(M=16, N=1040, K=512, dtype="bf16"),
}


@pytest.mark.parametrize("name", list(RSQ_CASES))
def test_row_sum_of_squares_matches_oracle(name):
    kw = dict(RSQ_CASES[name])
    if isinstance(kw.get("force"), str):
        kw["force"] = _index(kw["force"])
    c = Case(seed=300 + list(RSQ_CASES).index(name), row_sumsq=True, **kw)
    p = Prepared(c)
    g, out = p.run()
    assert b"skinny" not in g.info.name and g.workspace_bytes > 0
    got_d, _ = p.decode_out(out)
    assert error(c.dtype, got_d, p.oracle_full()) <= TOL[c.dtype]
    rsq = p.rsq.cpu().numpy().astype(np.float64)
    # the oracle's reduction: its double result rounded to the output type, squared, summed
    want = oracle.row_sumsq(p.oracle_full(), OUT_T[c.dtype])
    err = error("f32" if c.dtype == "f32" else c.dtype, rsq, want)
    print(f"{name}: {g.info.name.decode()} err={err:.3e}")
    assert err <= TOL[c.dtype], (name, err)


def test_row_sum_of_squares_is_exact_on_dyadic_inputs():
    # K = 16 dyadic products: every D value is a multiple of 1/16 of magnitude at most 16 (exact
    # in bf16), every square a multiple of 1/256 of at most 2^16 such units, and 256 of them stay
    # within 2^24 units, so the fp32 accumulation is exact and must equal the oracle's double sum
    # bit for bit
    c = Case(M=200, N=256, K=16, dtype="bf16", dist="dyadic", seed=310, row_sumsq=True)
    p = Prepared(c)
    g, out = p.run()
    want = oracle.row_sumsq(p.oracle_full(), "bf16")
    got = p.rsq.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want), (g.info.name.decode(), int((got != want).sum()))


@pytest.mark.parametrize("name", list(RSQ_CASES))
def test_column_sums_match_oracle(name):
    kw = dict(RSQ_CASES[name])
    if isinstance(kw.get("force"), str):
        kw["force"] = _index(kw["force"])
    both = list(RSQ_CASES).index(name) % 2 == 0     # every other case asks for both reductions
    c = Case(seed=320 + list(RSQ_CASES).index(name), col_sum=True, row_sumsq=both, **kw)
    p = Prepared(c)
    g, out = p.run()
    full = p.oracle_full()
    ot = OUT_T[c.dtype]
    cs = p.csum.cpu().numpy().astype(np.float64)
    want = oracle.col_sum(full, ot)
    # column sums of signed values can cancel: measure against the largest column sum of
    # magnitudes of the stored oracle values
    mag = oracle.col_sum(np.abs(full), ot).max()
    err = float(np.abs(cs - want).max() / mag)
    print(f"{name}: {g.info.name.decode()} err={err:.3e}")
    assert err <= TOL[c.dtype], (name, err)
    if both:
        rsq = p.rsq.cpu().numpy().astype(np.float64)
        assert error("f32" if c.dtype == "f32" else c.dtype, rsq, oracle.row_sumsq(full, ot)) <= TOL[c.dtype]


def test_column_sums_are_exact_on_dyadic_inputs():
    # K = 16 dyadic products: D values are multiples of 1/16 of magnitude at most 16 (exact in
    # bf16); 520 of them stay far within 2^24 units of 1/16 and 200 squares within 2^24 units of
    # 1/256, so both fp32 reductions equal the oracle bit for bit
    c = Case(M=520, N=200, K=16, dtype="bf16", dist="dyadic", seed=330, col_sum=True,
             row_sumsq=True)
    p = Prepared(c)
    g, out = p.run()
    full = p.oracle_full()
    got_cs = p.csum.cpu().numpy().astype(np.float64)
    got_rsq = p.rsq.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_cs, oracle.col_sum(full, "bf16")), g.info.name.decode()
    assert np.array_equal(got_rsq, oracle.row_sumsq(full, "bf16")), g.info.name.decode()
