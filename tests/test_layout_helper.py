"""The library's layout helper (C++, through the C ABI) against the pages' printed values and,
point by point, against the oracle's definitions (oracle.layout), bit-exact."""
import itertools
import json
import os
import random

import pytest

from hierarchical_tiling_amd import htgemm as H
from oracle import layout as L
from oracle import tile as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LP = json.load(open(os.path.join(GOLD, "layout_pins.json")))
TP = json.load(open(os.path.join(GOLD, "tile_pins.json")))


@pytest.mark.parametrize("pin", LP["eval"], ids=lambda p: f"{p['layout']}@{p['coord']}")
def test_eval_pins(pin):
    assert H.ht_layout_eval(pin["layout"], tuple(pin["coord"])) == pin["value"]


@pytest.mark.parametrize("pin", LP["tables_2d"], ids=lambda p: p["layout"])
def test_2d_tables(pin):
    rows = pin["rows"]
    got = [[H.ht_layout_eval(pin["layout"], (r, c)) for c in range(len(rows[0]))] for r in range(len(rows))]
    assert got == rows


def test_same_function_and_coalesce_pins():
    for pin in LP["same_function_1d"]:
        assert H.ht_layout_table(pin["a"]) == H.ht_layout_table(pin["b"])
        assert H.ht_layout_coalesce(pin["a"]) == pin["b"]
    for pin in LP["coalesce"]:
        assert H.ht_layout_coalesce(pin["layout"]) == pin["result"]
        assert H.ht_layout_coalesce("(_2,(_1,_6)):(_1,(_6,_2))") == "12:1"   # CuTe spelling


def test_compose_pin():
    for pin in LP["compose"]:
        r = H.ht_layout_compose(pin["a"], pin["b"])
        assert r == pin["result"]
        assert H.ht_layout_table(r) == L.compose_table(L.parse(pin["a"]), L.parse(pin["b"]))


@pytest.mark.parametrize("pin", LP["complement"], ids=lambda p: f"{p['layout']}|{p['size']}")
def test_complement_pins(pin):
    assert H.ht_layout_complement(pin["layout"], pin["size"]) == pin["result"]


def test_logical_divide_pin():
    for pin in LP["logical_divide"]:
        assert H.ht_layout_logical_divide(pin["a"], pin["b"]) == pin["result"]


def test_swizzle_pin_and_definition():
    pin = LP["swizzle_bank"][0]
    for c in range(pin["cols"]):
        offs = [H.ht_swizzle(r * pin["cols"] + c, pin["bbits"], pin["mbase"], pin["sshift"]) for r in range(pin["rows"])]
        assert len(L.bank_set(offs, pin["banks"])) == pin["distinct_banks_per_column_swizzled"]
    rng = random.Random(5)
    for _ in range(2000):
        o, b, m, s = rng.randrange(1 << 20), rng.randrange(1, 6), rng.randrange(0, 5), rng.randrange(1, 8)
        assert H.ht_swizzle(o, b, m, s) == L.swizzle(o, b, m, s)


def test_tile_plan_pins():
    w = TP["tile_widget"]
    for kib in w["budget_kib"]:
        st = H.ht_tile_plan(w["m"], w["n"], w["k"], w["bytes_per_elem"], kib * 1024)
        assert st.flops == w["flops"]
        assert f"{st.intensity:.2f}" == w["intensity_flop_per_byte_2dp"]
        assert bool(st.fits) == w["buffers_fit"]
        assert st.bytes == T.tile_bytes(w["m"], w["n"], w["k"], w["bytes_per_elem"])
        assert st.double_buffer_bytes == T.double_buffer_bytes(w["m"], w["n"], w["k"], w["bytes_per_elem"])
    assert not H.ht_tile_plan(256, 256, 64, 2, 64 * 1024).fits   # 128 KiB of double buffers
    p = TP["pipeline_widget"]
    assert H.ht_pipeline_time(p["tiles"], p["load_us"], p["compute_us"]) == p["pipelined_us"]
    assert H.ht_pipeline_time(0, 4.0, 6.0) == 0.0


def test_errors():
    with pytest.raises(H.LayoutError) as e:
        H.ht_layout_eval("(4,3):(3,1)", (4, 0))
    assert e.value.status == 2
    with pytest.raises(H.LayoutError) as e:
        H.ht_layout_eval("(4,3):(3", (0, 0))
    assert e.value.status == 1
    with pytest.raises(H.LayoutError) as e:
        H.ht_layout_compose("(6,2):(8,2)", "3:4")           # stride 4 does not divide through 6
    assert e.value.status == 3
    with pytest.raises(H.LayoutError) as e:
        H.ht_layout_coalesce("(4,3:(3,1)")
    assert e.value.status == 1


# ---- properties against the oracle's definitions on random layouts ------------------------

def rand_layout(rng, max_modes=3, nested=True):
    n = rng.randint(1, max_modes)
    shape = [rng.choice([1, 2, 3, 4, 6, 8]) for _ in range(n)]
    stride = [rng.choice([0, 1, 2, 3, 4, 8, 16, 24]) for _ in range(n)]
    if nested and n >= 2 and rng.random() < 0.4:
        s = (tuple(shape[:2]),) + tuple(shape[2:])
        d = (tuple(stride[:2]),) + tuple(stride[2:])
    elif n == 1:
        s, d = shape[0], stride[0]
    else:
        s, d = tuple(shape), tuple(stride)
    return L.fmt(s, d)


def test_eval_table_matches_definition_on_random_layouts():
    rng = random.Random(1)
    for _ in range(400):
        lay = rand_layout(rng)
        assert H.ht_layout_table(lay) == L.table(L.parse(lay)), lay


def test_coalesce_keeps_the_function_and_is_minimal():
    rng = random.Random(2)
    for _ in range(400):
        lay = rand_layout(rng, 4)
        c = H.ht_layout_coalesce(lay)
        assert H.ht_layout_table(c) == L.table(L.parse(lay)), (lay, c)
        s, d = L.parse(c)
        fs, fd = L.flatten(s), L.flatten(d)
        assert all(x != 1 for x in fs) or fs == (1,)
        for i in range(len(fs) - 1):
            assert fd[i + 1] != fs[i] * fd[i], (lay, c)


def test_compose_matches_definition_on_random_compact_layouts():
    rng = random.Random(3)
    checked = 0
    for _ in range(3000):
        # A: a permutation-like compact layout; B: any layout into A's domain
        n = rng.randint(1, 3)
        shp = [rng.choice([2, 3, 4]) for _ in range(n)]
        order = list(range(n))
        rng.shuffle(order)
        strides = [0] * n
        acc = 1
        for i in order:
            strides[i] = acc
            acc *= shp[i]
        a = L.fmt(tuple(shp) if n > 1 else shp[0], tuple(strides) if n > 1 else strides[0])
        size_a = acc
        bs = rng.choice([1, 2, 3, 4, 6])
        bd = rng.choice([1, 2, 3, 4, 6])
        b2 = rng.choice([1, 2, 3])
        b = f"({bs},{b2}):({bd},{bd * bs})"
        if (bs * b2 - 1) * bd >= size_a * 4:
            continue
        try:
            r = H.ht_layout_compose(a, b)
        except H.LayoutError as e:
            assert e.status == 3
            continue
        la, lb = L.parse(a), L.parse(b)
        if max(L.table(lb)) >= size_a:
            continue  # beyond A's domain the last mode is extended; not a definition case
        assert H.ht_layout_table(r) == L.compose_table(la, lb), (a, b, r)
        assert L.compatible(L.parse(r), lb)
        checked += 1
    assert checked > 200


def test_complement_matches_brute_force():
    rng = random.Random(4)
    checked = 0
    for _ in range(500):
        s = rng.choice([2, 3, 4, 6])
        d = rng.choice([1, 2, 3, 4, 8])
        m = s * d * rng.choice([1, 2, 3, 4])
        lay = f"{s}:{d}"
        want = L.complement_brute(L.parse(lay), m)
        try:
            got = H.ht_layout_complement(lay, m)
        except H.LayoutError:
            assert want is None
            continue
        if want is None:
            continue
        assert L.table(L.parse(got)) == L.table(want), (lay, m, got)
        checked += 1
    assert checked > 100


def test_logical_and_zipped_divide_match_definition():
    rng = random.Random(6)
    for _ in range(200):
        t = rng.choice([2, 4])
        ts = rng.choice([1, 2])
        a = rng.choice(["(4,2,3):(2,1,8)", "24:1", "(8,3):(3,1)", "(4,6):(1,4)"])
        b = f"{t}:{ts}"
        r = H.ht_layout_logical_divide(a, b)
        la, lb = L.parse(a), L.parse(b)
        comp = L.complement_brute(lb, L.size(la[0]))
        if comp is None:
            continue
        concat = ((lb[0], comp[0]), (lb[1], comp[1]))
        assert H.ht_layout_table(r) == L.compose_table(la, concat), (a, b, r)
    # zipped_divide of a 2-D layout: ((tile0,tile1),(rest0,rest1))
    z = H.ht_layout_zipped_divide("(8,12):(1,8)", "4:1", "3:1")
    zl = L.parse(z)
    assert L.top_sizes(zl) == (12, 8)
    m0, m1 = L.parse("8:1"), L.parse("12:8")
    for i0 in range(4):
        for i1 in range(3):
            for r0 in range(2):
                for r1 in range(4):
                    want = L.evaluate(m0, i0 + 4 * r0) + L.evaluate(m1, i1 + 3 * r1)
                    assert L.evaluate(zl, ((i0, i1), (r0, r1))) == want


def _view_table(off, text, sizes):
    """Offsets of a helper view at every coordinate (one 1-D index per top-level mode)."""
    lay = L.parse(text)
    out = []
    for c in itertools.product(*[range(s) for s in sizes]):
        out.append(off + L.evaluate(lay, c if len(c) > 1 else c[0]))
    return out


def test_local_tile_matches_oracle():
    rng = random.Random(11)
    layouts = ["(8,12):(12,1)", "(8,12):(1,8)", "((2,4),12):((1,24),2)", "(8,6,3):(6,1,48)",
               "(16,(2,6)):(1,(16,32))"]
    checked = 0
    for _ in range(300):
        a = rng.choice(layouts)
        la = L.parse(a)
        sz = L.top_sizes(la)
        t0 = rng.choice([d for d in (1, 2, 4, 8) if sz[0] % d == 0])
        t1 = rng.choice([d for d in (1, 2, 3, 4, 6, 12) if sz[1] % d == 0])
        tiler = (t0, t1)
        rest = (sz[0] // t0, sz[1] // t1) + sz[2:]
        coord = tuple(None if rng.random() < 0.4 else rng.randrange(r) for r in rest)
        try:
            off, text = H.ht_layout_local_tile(a, tiler, coord)
        except H.LayoutError as e:
            # composition needs each tile size to divide, or be a multiple of, the size of the
            # first sub-mode it enters: 3:1 into (2,6) does neither
            first = [m[0][0] if isinstance(m[0], tuple) else m[0] for m in L._modes(la)]
            assert e.status == 3 and any(t % f and f % t for t, f in zip(tiler, first))
            continue
        sizes, g = L.local_tile(la, tiler, coord)
        assert L.top_sizes(L.parse(text)) == sizes, (a, tiler, coord, text)
        want = [g(c) for c in itertools.product(*[range(s) for s in sizes])]
        assert _view_table(off, text, sizes) == want, (a, tiler, coord, off, text)
        checked += 1
    assert checked > 250


def test_local_tile_projection_matches_oracle():
    a, tiler, coord = "(8,6):(6,1)", (4, 3, 2), (1, 2, None)
    for proj in (("1", "X", "1"), "(1,X,1)"):
        off, text = H.ht_layout_local_tile(a, tiler, coord, proj)
        sizes, g = L.local_tile(L.parse(a), tiler, coord, ("1", "X", "1"))
        assert (off, text) == (6 * 4, "(4,2,3):(6,1,2)")
        assert _view_table(off, text, sizes) == [g(c) for c in itertools.product(*map(range, sizes))]


def test_local_partition_matches_oracle():
    cases = [("64:1", (32,)), ("(16,64):(64,1)", (2, 16)), ("(8,12):(1,8)", (4, 3)),
             ("((2,4),6):((6,1),12)", (2, 3)), ("(8,6,3):(6,1,48)", (2, 2))]
    for a, thr in cases:
        n = 1
        for t in thr:
            n *= t
        for idx in range(n):
            off, text = H.ht_layout_local_partition(a, thr, idx)
            sizes, g = L.local_partition(L.parse(a), thr, idx)
            assert L.top_sizes(L.parse(text)) == sizes, (a, thr, idx, text)
            want = [g(c) for c in itertools.product(*[range(s) for s in sizes])]
            assert _view_table(off, text, sizes) == want, (a, thr, idx)


@pytest.mark.parametrize("call,code", [
    (lambda: H.ht_layout_local_tile("(8,12):(12,1)", (3, 3), (0, None)), 3),   # 3 does not divide 8
    (lambda: H.ht_layout_local_tile("(8,12):(12,1)", (4, 3), (2, None)), 2),   # 2 row blocks only
    (lambda: H.ht_layout_local_tile("(8,12):(12,1)", (4, 3), (0,)), 2),        # rank mismatch
    (lambda: H.ht_layout_local_tile("(8,12):(12,1)", (4, 3, 2), (0, 0, 0), "(1,X)"), 2),
    (lambda: H.ht_layout_local_tile("(8,12):(12,1)", "(4,_)", (0, 0)), 1),     # "_" is no tile size
    (lambda: H.ht_layout_local_partition("(8,12):(12,1)", (4, 3), 12), 2),     # threads 0 .. 11
    (lambda: H.ht_layout_local_partition("(8,12):(12,1)", (3, 3), 0), 3),
])
def test_local_tile_and_partition_errors(call, code):
    with pytest.raises(H.LayoutError) as e:
        call()
    assert e.value.status == code


def test_eval_through_the_c_abi_with_integer_coordinates():
    # the boundary's own form: a caller-owned int64 array and its rank ("CUTLASS, CuTe, and CUDA
    # Tile", introduction: (4,3):(3,1) maps (1,0) to 3 and (0,1) to 1)
    import ctypes
    L = H.lib()
    out = ctypes.c_int64()

    def ev(layout, coord):
        arr = (ctypes.c_int64 * len(coord))(*coord)
        rc = L.ht_layout_eval(layout.encode(), arr, len(coord), ctypes.byref(out))
        return rc, out.value

    assert ev("(4,3):(3,1)", [1, 0]) == (0, 3)
    assert ev("(4,3):(3,1)", [0, 1]) == (0, 1)
    # rank 1 is a 1-D coordinate (leftmost mode fastest): 5 -> (1, 1) -> 3 + 1
    assert ev("(4,3):(3,1)", [5]) == (0, 4)
    # one integer per top-level mode of a nested layout: the composition pin's element 11
    assert ev("((2,2),3):((24,2),8)", [3, 2]) == (0, 42)
    assert ev("(4,3):(3,1)", [4, 0])[0] == 2        # outside the shape: HT_ERR_RANGE
    assert ev("(4,3):(3,1)", [1, 0, 0])[0] == 2     # rank is neither 1 nor the mode count
    assert ev("(4,3):(3", [0, 0])[0] == 1           # bad text: HT_ERR_PARSE
