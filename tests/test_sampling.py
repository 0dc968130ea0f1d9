"""The sampled oracle used at full problem sizes gives exactly the full oracle's values at the
sampled places (host only: the inputs stay on the CPU and no kernel runs)."""
import numpy as np
import pytest

from tests.gemm_util import Case, Prepared


@pytest.mark.parametrize("case", [
    Case(37, 29, 23, "bf16", has_c=True, beta=-0.5, bias=True, act="gelu", seed=3),
    Case(40, 33, 17, "f16", "col", "row", a_ld=45, b_ld=35, has_c=True, beta=1.25, alpha=0.75,
         row_scale=True, col_scale=True, seed=4),
    Case(16, 70, 64, "e4m3", std=1.0, scale_a=0.05, scale_b=0.05, seed=5),
    Case(9, 8, 5, "f32", "row", "row", dist="uniform", has_c=True, beta=0.5, alpha=1.5, seed=6),
])
def test_sample_equals_full_oracle(case):
    p = Prepared(case, device="cpu")
    full = p.oracle_full()
    # the "device result" here is the oracle itself: the sample must pick the same places
    have, want, what = p.oracle_sample(full, seed=1, n_rows=6, n_cols=5, n_rand=50)
    assert np.array_equal(have, want), what
    assert str(min(case.M, 6)) in what


def test_sample_picks_first_and_last_rows_and_columns():
    p = Prepared(Case(50, 60, 8, "bf16", seed=7), device="cpu")
    full = p.oracle_full()
    marked = full.copy()
    marked[0, :] = marked[-1, :] = marked[:, 0] = marked[:, -1] = np.nan
    have, _, _ = p.oracle_sample(marked, seed=2, n_rows=4, n_cols=4, n_rand=10)
    # both edge rows (2 x 60 values) and both edge columns (2 x 50) are in the sample
    assert np.isnan(have).sum() >= 2 * 60 + 2 * 50 - 4
