"""GPU parity of the ping-pong kernel (two groups of four waves taking turns between MFMA and
LDS/DMA phases) through its table entries, forced, against the CPU oracle.

The kernel's phase schedule depends on the number of k-tiles (its prologue loads two of them, its
loop issues loads two ahead, zero-filled past K), so the cases run one, two and three k-tiles
with partial last ones, ragged M and N edges, a K split and the fused epilogue extras; dyadic
inputs must match the oracle bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error

pytestmark = pytest.mark.gpu

PP = {"bf16": "bf16_ak_bk_256x256x64_w2x4_m16_pp", "f16": "f16_ak_bk_256x256x64_w2x4_m16_pp",
      "e4m3": "e4m3_ak_bk_256x256x128_w2x4_m16_pp", "bf16_bn": "bf16_ak_bn_256x256x64_w2x4_m16_pp",
      "f16_bn": "f16_ak_bn_256x256x64_w2x4_m16_pp"}


def _index(name):
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())].index(name)


def _case(key, M, N, K, **kw):
    dtype = key.split("_")[0]
    b_order = "row" if key.endswith("_bn") else "col"
    extra = dict(std=1.0, scale_a=0.5, scale_b=0.25) if dtype == "e4m3" else {}
    extra.update(kw)
    return Case(M, N, K, dtype, "row", b_order, force=_index(PP[key]), split_k=1, **extra)


def _check(c, expect_split=1):
    p = Prepared(c)
    g, out = p.run()
    assert g.info.name.decode() == H.gemm_config_name(c.force)
    assert g.info.split_k == expect_split
    got, bits = p.decode_out(out)
    want = p.oracle_full()
    if c.dist == "dyadic":
        mism = int((bits != oracle.encode_rne(OUT_T[c.dtype], want)).sum())
        assert mism == 0, f"{mism} of {bits.size} outputs differ"
        return
    assert np.isfinite(got).all()
    err = error(c.dtype, got, want)
    print(f"{g.info.name.decode()} {c.M}x{c.N}x{c.K}: err={err:.3e}")
    assert err <= TOL[c.dtype], err


# k-tiles of 64 (2-byte) or 128 (fp8) elements: one partial, two, three with a partial last
DEPTHS = {"bf16": (40, 128, 136), "f16": (40, 128, 136), "e4m3": (48, 256, 272)}


@pytest.mark.parametrize("key", list(PP))
@pytest.mark.parametrize("depth", [0, 1, 2])
def test_short_k_and_ragged_edges(key, depth):
    K = DEPTHS[key.split("_")[0]][depth]
    c = _case(key, 300, 520, K, has_c=True, beta=-0.5, alpha=0.75, bias=True, act="gelu",
              seed=600 + 3 * list(PP).index(key) + depth)
    _check(c)


@pytest.mark.parametrize("key", list(PP))
def test_dyadic_bit_exact(key):
    c = _case(key, 520, 264, 2 * DEPTHS[key.split("_")[0]][2], dist="dyadic", alpha=2.0, beta=0.5,
              has_c=True, bias=True, seed=620 + list(PP).index(key))
    _check(c)


@pytest.mark.parametrize("key", ["bf16", "e4m3", "bf16_bn"])
def test_k_split(key):
    # three K slices through the fp32 planes and the sum kernel (N a multiple of 8: the 16-byte
    # loads of a row-major B)
    c = _case(key, 264, 296, 3 * DEPTHS[key.split("_")[0]][2], has_c=True, beta=0.5, bias=True,
              act="relu", seed=630 + list(PP).index(key))
    _check(dataclasses.replace(c, split_k=3), expect_split=3)


@pytest.mark.parametrize("key", ["bf16", "f16_bn"])
def test_epilogue_extras(key):
    # per-row and per-column scale vectors and SiLU from the ping-pong kernel's accumulators
    c = _case(key, 300, 280, 200, bias=True, act="silu", row_scale=True, col_scale=True,
              seed=640 + list(PP).index(key))
    _check(c)


def test_same_bits_as_the_split_ring():
    # the two kernels sum each output in the same order, so they agree bit for bit on any input
    for key, ring in (("bf16", "bf16_ak_bk_256x256x64_w2x4_m16_ring"),
                      ("bf16_bn", "bf16_ak_bn_256x256x64_w2x4_m16_ring")):
        c = _case(key, 1000, 1304, 1000, bias=True, act="gelu", seed=650)
        p = Prepared(c)
        _, out = p.run()
        _, bits_pp = p.decode_out(out)
        p2 = Prepared(dataclasses.replace(c, force=_index(ring)))
        _, out2 = p2.run()
        _, bits_ring = p2.decode_out(out2)
        assert int((bits_pp != bits_ring).sum()) == 0, key


@pytest.mark.parametrize("key", ["bf16", "e4m3", "f16_bn"])
def test_plain_epilogue_copy_matches_the_general_one(key):
    # launches without C, scale vectors or fused reductions, D in whole 16-byte rows, take the
    # epilogue copy compiled for them; a row scale of ones sends the same product through the
    # general copy (a multiply by one is exact), which must give the same bits
    dtype = key.split("_")[0]
    c = _case(key, 520, 600, DEPTHS[dtype][2] * 3, bias=True, act="gelu",
              seed=670 + list(PP).index(key))
    p = Prepared(c)
    _, out = p.run()
    _, bits_plain = p.decode_out(out)
    p2 = Prepared(dataclasses.replace(c, row_scale=True))
    p2.rs = np.ones(c.M, dtype=np.float32)
    p2.drs = torch.ones(c.M, dtype=torch.float32, device=p2.device)
    _, out2 = p2.run()
    _, bits_general = p2.decode_out(out2)
    assert int((bits_plain != bits_general).sum()) == 0, key
    _check(c)


@pytest.mark.parametrize("key", ["bf16", "e4m3", "f16_bn"])
def test_padded_leading_dimensions(key):
    # rows of A and B (and of C and D) longer than the product reads: the DMA's row strides and
    # range checks use the leading dimensions, not K or N (each a multiple of 16 bytes)
    dtype = key.split("_")[0]
    K = DEPTHS[dtype][2] * 2
    pad = 16 if dtype == "e4m3" else 8
    b_ld = (520 + 3 * pad) if key.endswith("_bn") else K + 5 * pad
    c = _case(key, 300, 520, K, a_ld=K + 3 * pad, b_ld=b_ld, c_ld=536, d_ld=544, has_c=True,
              beta=0.25, bias=True, act="gelu", seed=660 + list(PP).index(key))
    _check(c)


def test_clock_record():
    # the opt-in clock record: every workgroup of the launch writes its shader-clock and
    # real-time counters at start and end; the product is unchanged, and turning the record off
    # leaves the buffer alone
    import torch
    c = _case("bf16", 520, 776, 512, bias=True, act="gelu", seed=670)
    p = Prepared(c)
    g, out = p.run()
    n = int(g.info.grid)
    assert n == 3 * 4
    rec = torch.zeros(4 * n + 4, dtype=torch.int64, device="cuda")
    H.gemm_set_clock_record(g.handle, rec, n)
    g2, out2 = p.run(g=g)
    torch.cuda.synchronize()
    r = rec.cpu().numpy().reshape(-1, 4)
    assert (r[n] == 0).all(), "a workgroup past max_workgroups wrote"
    r = r[:n].astype(np.float64)
    assert (r[:, 1] > r[:, 0]).all() and (r[:, 3] > r[:, 2]).all()
    mhz = (r[:, 1] - r[:, 0]) / (r[:, 3] - r[:, 2]) * 100.0
    print(f"clock record: {np.median(mhz):.0f} MHz median over {n} workgroups")
    assert ((mhz > 100) & (mhz < 3000)).all(), mhz
    got, _ = p.decode_out(out2)
    assert error("bf16", got, p.oracle_full()) <= TOL["bf16"]
    H.gemm_set_clock_record(g.handle, None, 0)
    rec.zero_()
    p.run(g=g)
    torch.cuda.synchronize()
    assert int(rec.abs().sum()) == 0
