"""The cost model behind the kernel choice (host only): every tiled entry has measured costs,
the library's prediction follows the measured table by the same formula as the calibration
script's, and the automatic choice is the fitting entry with the least predicted time."""
import os
import re

import pytest

from hierarchical_tiling_amd import calibrate as C
from hierarchical_tiling_amd import htgemm as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "hierarchical_tiling_amd", "csrc", "cost_table.cpp")


@pytest.fixture
def fake_gfx950(monkeypatch):
    monkeypatch.setenv("HTGEMM_FAKE_ARCH", "gfx950")


def _floats(text):
    return [float(x.strip().rstrip("f")) for x in text.split(",") if x.strip()]


def table(with_edges=False):
    """(per-entry [(f, c)] at the measured loads, {constant name: value}) read from the source;
    with_edges adds {entry: (partial k-tile cost, partial tile row/column cost)}."""
    text = open(TABLE).read()
    rows, edges = {}, {}
    num = r"\s*([-0-9.]+)f"
    for m in re.finditer(r'\{"([^"]+)",\s*\{([^}]*)\},\s*\{([^}]*)\},' + num + "," + num + "," + num + r"\}",
                         text):
        f, c = _floats(m.group(2)), _floats(m.group(3))
        assert len(f) == len(c) == len(C.LOADS), m.group(1)
        rows[m.group(1)] = list(zip(f, c))
        edges[m.group(1)] = tuple(float(m.group(i)) for i in (4, 5, 6))
    consts = {m.group(1): float(m.group(2))
              for m in re.finditer(r"const double (k\w+) = ([-+0-9.e]+);", text)}
    return (rows, consts, edges) if with_edges else (rows, consts)


def info(d):
    h = H.gemm_create(d)
    try:
        return H.gemm_get_info(h)
    finally:
        H.gemm_destroy(h)


def names():
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]


def test_every_tiled_entry_has_costs():
    rows, consts = table()
    tiled = {n for n in names() if C.parse_name(n)[3] != "skinny"}
    assert tiled == set(rows), (tiled ^ set(rows))
    for name, r in rows.items():
        assert all(f >= 0 and c > 0 for f, c in r), name
    for k in ("kSplitFixedUs", "kSplitUsPerByte", "kRepackFixedUs", "kRepackUsPerByte",
              "kSkFixedUs", "kSkShareFactor"):
        assert k in consts and consts[k] >= 0


def _forced(name, M, N, K, split_k=1, decomposition=1):
    dtype, ak, bk, _ = C.parse_name(name)
    a = (K, 1) if ak else (1, M)
    b = (1, K) if bk else (N, 1)
    return H.make_desc(M, N, K, dtype, a, b, (N, 1), force_config=names().index(name),
                       split_k=split_k, decomposition=decomposition)


@pytest.mark.parametrize("name", ["bf16_ak_bk_256x256x64_w2x4_m16_ring",
                                  "bf16_ak_bk_128x128x64_w2x2_m32_vec",
                                  "f16_ak_bn_64x64x64_w2x2_m16_vec",
                                  "e4m3_ak_bk_256x256x128_w2x4_m32_ring",
                                  "f32_am_bk_128x128x32_w2x2_m32_vec"])
@pytest.mark.parametrize("tiles_mn,kt", [((8, 8), 16), ((8, 16), 40), ((16, 16), 64), ((16, 19), 7),
                                         ((32, 32), 128), ((32, 64), 9), ((48, 48), 33),
                                         ((10, 13), 100)])
def test_prediction_follows_the_table(fake_gfx950, name, tiles_mn, kt):
    """A forced, unsplit run: the prediction is the table's f + kt * c at whole loads, and the
    calibration script's formula between them (partial last rounds, loads above 8)."""
    rows, _ = table()
    i = info(_forced(name, 256, 256, 512))
    bm, bn, bk = i.bm, i.bn, i.bk
    tm, tn = tiles_mn
    got = info(_forced(name, tm * bm, tn * bn, kt * bk))
    assert got.split_k == 1 and got.sk_tiles == 0 and got.tail_tiles == 0
    want = C.predict(rows[name], tm * tn, kt)
    assert got.predicted_us == pytest.approx(want, rel=1e-5)
    if tm * tn in (256, 1024, 2048):
        n = tm * tn // 256
        f, c = rows[name][C.LOADS.index(n)]
        assert got.predicted_us == pytest.approx(f + kt * c, rel=1e-5)


@pytest.mark.parametrize("name", ["bf16_ak_bk_256x256x64_w2x4_m16_ring",
                                  "f16_ak_bk_128x128x64_w2x2_m32_narrow",
                                  "e4m3_ak_bn_64x64x128_w2x2_m16_narrow"])
def test_prediction_of_partial_edges(fake_gfx950, name):
    """A partial last k-tile and D rows off 16 bytes add their measured costs once per workgroup
    on the busiest compute unit; partial last tile rows or columns add theirs once."""
    rows, _, edges = table(with_edges=True)
    i = info(_forced(name, 256, 256, 512))
    bm, bn, bk = i.bm, i.bn, i.bk
    M, N, kt = 20 * bm, 16 * bn, 24   # 320 tiles: two workgroups on the busiest unit
    base = C.predict(rows[name], 320, kt)
    ek, emn, ed = edges[name]
    k_edge = info(_forced(name, M, N, kt * bk - bk // 2))
    assert k_edge.predicted_us == pytest.approx(base + 2 * ek, rel=1e-5)
    mn_edge = info(_forced(name, M - bm + 8, N - 8, kt * bk))
    assert mn_edge.predicted_us == pytest.approx(base + emn, rel=1e-5)
    odd_d = _forced(name, M, N, kt * bk)
    odd_d.d_stride_m = N + 1
    assert info(odd_d).predicted_us == pytest.approx(base + 2 * ed, rel=1e-5)
    assert C.edge_time(edges[name], M - bm + 8, N - 8, kt * bk - bk // 2, bm, bn, bk,
                       d_rows_aligned=False) == pytest.approx(2 * ek + emn + 2 * ed)


def test_prediction_of_stream_k_and_split(fake_gfx950):
    """Stream-K: whole tiles, then the fitted cost of 256 workgroups' shares; a forced split: the
    launch of tiles x S workgroups plus the sum kernel over the fp32 planes."""
    rows, k = table()
    ring = "bf16_ak_bk_256x256x64_w2x4_m16_ring"
    r = rows[ring]
    sk = info(_forced(ring, 17 * 256, 18 * 256, 64 * 64, split_k=0, decomposition=2))
    tiles = 17 * 18
    assert sk.sk_tiles == tiles - 256
    want = (C.predict(r, 256, 64) + k["kSkFixedUs"] +
            k["kSkShareFactor"] * C.predict(r, 256, -(-(tiles - 256) * 64 // 256)))
    assert sk.predicted_us == pytest.approx(want, rel=1e-5)
    M = N = 1536
    sp = info(_forced(ring, M, N, 8192, split_k=4))
    assert sp.split_k == 4
    want = (C.predict(r, 36 * 4, 32) + k["kSplitFixedUs"] +
            k["kSplitUsPerByte"] * (2 * 4 * M * N * 4 + M * N * 2))
    assert sp.predicted_us == pytest.approx(want, rel=1e-5)


@pytest.mark.parametrize("dtype,M,N,K,bk", [
    ("bf16", 3072, 3072, 3072, True), ("bf16", 1536, 1536, 8192, True),
    ("bf16", 4352, 4352, 4096, True), ("bf16", 704, 896, 1088, True),
    ("bf16", 4096, 4096, 4096, False), ("f16", 2048, 1024, 512, True),
    ("e4m3", 4096, 4096, 8192, True), ("f32", 1000, 1000, 1000, True),
])
def test_choice_is_the_least_predicted(fake_gfx950, dtype, M, N, K, bk):
    """The automatic choice is predicted within 3 % (the tie tolerance) of the least predicted
    time of all entries that fit, each under the plan it would get; among the entries in that
    band it has the least sustained cost (per-k-tile time at four workgroups per compute unit,
    per multiply-add of a k-tile)."""
    rows, _ = table()
    b = (1, K) if bk else (N, 1)
    auto = info(H.make_desc(M, N, K, dtype, (K, 1), b, (N, 1)))
    assert auto.predicted_us > 0
    preds = {}
    for i, name in enumerate(names()):
        d_, ak_, bk_, kind = C.parse_name(name)
        if d_ != dtype or not ak_ or bk_ != bk or kind in ("skinny", "narrow", "realign"):
            continue
        try:
            preds[name] = info(H.make_desc(M, N, K, dtype, (K, 1), b, (N, 1), force_config=i))
        except H.GemmError:
            continue   # the entry does not fit this product
    least = min(p.predicted_us for p in preds.values())
    assert auto.predicted_us <= least * 1.03 * (1 + 1e-9)

    def sustained(p):
        return rows[p.name.decode()][C.LOADS.index(4)][1] / (p.bm * p.bn * p.bk)
    band = [p for p in preds.values() if p.predicted_us <= least * 1.03 * (1 + 1e-9)]
    assert sustained(auto) == pytest.approx(min(sustained(p) for p in band), rel=1e-6)
