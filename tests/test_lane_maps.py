"""The MFMA atoms' lane maps as layouts (host only).

"A10 - CuTe, CUTLASS & CuTile", section 3.3: an MMA atom's A, B and C fragments are layouts from
(thread, value) to the instruction's tile, and their per-thread counts close exactly over the
tile; section 6 Pitfall 2: a wrong fragment map gives silently wrong results.  Here each map of
tests/golden/lane_maps.json is evaluated by the layout helper and by the oracle's pointwise
definition, must be a bijection onto its tile with the pages' closure arithmetic, must put lane l
on row / column l % MI, and must be exactly the layout the library's kernels were built with.
"""
import json
import os

import pytest

from hierarchical_tiling_amd import htgemm as H
from oracle import layout as OL

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lane_maps.json")))
ATOMS = GOLDEN["atoms"]


def _id(a):
    return f"{a['dtype']}_{a['mi']}"


@pytest.mark.parametrize("atom", ATOMS, ids=_id)
def test_closure_and_bijection(atom):
    mi, ki = atom["mi"], atom["ki"]
    op = H.ht_layout_table(atom["op"])
    acc = H.ht_layout_table(atom["acc"])
    # 64 lanes x values per lane cover the tile exactly once
    assert len(op) == 64 * atom["op_per_lane"] == mi * ki
    assert sorted(op) == list(range(mi * ki))
    assert len(acc) == 64 * atom["acc_per_lane"] == mi * mi
    assert sorted(acc) == list(range(mi * mi))
    # the helper and the oracle's pointwise definition agree on every slot
    assert op == OL.table(OL.parse(atom["op"]))
    assert acc == OL.table(OL.parse(atom["acc"]))


@pytest.mark.parametrize("atom", ATOMS, ids=_id)
def test_lane_l_owns_row_l_mod_mi(atom):
    mi = atom["mi"]
    op = H.ht_layout_table(atom["op"])
    acc = H.ht_layout_table(atom["acc"])
    for i, off in enumerate(op):
        assert off % mi == (i % 64) % mi            # operand row (A) / column (B)
    for i, off in enumerate(acc):
        assert off // mi == (i % 64) % mi           # accumulator column


def test_closure_pins():
    pins = GOLDEN["closure_pins"]
    by = {(a["dtype"], a["mi"]): a for a in ATOMS}
    a = by[("bf16", 16)]
    assert H.ht_layout_size(a["op"]) == pins["bf16_16x16x32"]["a_elements"] == 64 * 8
    assert a["op_per_lane"] == pins["bf16_16x16x32"]["a_per_lane"]
    assert H.ht_layout_size(a["acc"]) == pins["bf16_16x16x32"]["c_elements"] == 64 * 4
    b = by[("bf16", 32)]
    assert H.ht_layout_size(b["acc"]) == pins["bf16_32x32x16"]["c_elements"] == 64 * 16
    e = by[("e4m3", 16)]
    assert H.ht_layout_size(e["op"]) == pins["e4m3_16x16x128"]["a_elements"]
    assert e["op_per_lane"] * 1 == pins["e4m3_16x16x128"]["a_bytes_per_lane"]


@pytest.mark.parametrize("atom", ATOMS, ids=_id)
def test_library_kernels_use_these_layouts(atom):
    # the strings the kernels' compile-time tables were written from, which the library checks
    # against the helper itself (GEMM_ERR_LANE_MAP otherwise)
    op, acc = H.gemm_atom_layouts(atom["dtype"], atom["mi"])
    assert (op, acc) == (atom["op"], atom["acc"])


def test_unknown_atom_is_refused():
    with pytest.raises(H.GemmError):
        H.gemm_atom_layouts("bf16", 8)
