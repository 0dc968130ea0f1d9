"""Device index probe: where the hardware puts each MFMA value, against the layout helper's
evaluation of the atom's layouts, bit for bit ("A10 - CuTe, CUTLASS & CuTile", section 3.3 and
drill answer 4: the (thread, value) -> (m, n) map of a fragment; section 6 Pitfall 2)."""
import json
import os

import numpy as np
import pytest
import torch

from hierarchical_tiling_amd import htgemm as H

pytestmark = pytest.mark.gpu

ATOMS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lane_maps.json")))["atoms"]


@pytest.mark.parametrize("atom", ATOMS, ids=lambda a: f"{a['dtype']}_{a['mi']}")
def test_probe_matches_helper(atom):
    mi, nacc, vpl = atom["mi"], atom["acc_per_lane"], atom["op_per_lane"]
    out = torch.full((H.GEMM_PROBE_INTS,), -7, dtype=torch.int32, device="cuda")
    H.gemm_probe_atom(atom["dtype"], mi, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    acc = np.array(H.ht_layout_table(atom["acc"]))
    op = np.array(H.ht_layout_table(atom["op"]))
    n_acc, n_op = 64 * nacc, 64 * vpl
    # accumulator placement measured through the kernels' LDS tiles and fragment reads
    assert np.array_equal(o[:n_acc], acc), "hardware accumulator map differs from the layout"
    # the kernels' own accumulator positions
    assert np.array_equal(o[2048:2048 + n_acc], acc), "kernels' accumulator map differs"
    # the row of A each operand slot feeds, measured with one-hot inputs
    assert np.array_equal(o[4096:4096 + n_op], op % mi), "hardware operand rows differ"
    # slots the layout labels with the same k meet in the hardware's product for every column
    assert np.array_equal(o[6144:6144 + n_op], np.full(n_op, mi)), "k labels do not meet"
    # nothing written past the atom's slots
    assert (o[n_acc:2048] == -2).all() and (o[4096 + n_op:6144] == -2).all()
