"""Large products whose operands the 16-byte loaders cannot read run on aligned K-major copies of
A and B made in the workspace (gemm_info.repack), then on the aligned kernels.  Parity against the
oracle, including K not a multiple of 8 (the copies are zero-padded), every storage order with
odd leading dimensions, fp8 with row-major B, C, bias and GELU; the dyadic case bit for bit."""
import numpy as np
import pytest

import oracle
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error

pytestmark = pytest.mark.gpu

# The cost model decides whether to copy (copies plus the kernel chosen for them against the best
# direct entry); each case here is one it runs on copies.
CASES = {
    # fp16, odd leading dimensions in every operand, B row-major, C and GELU
    "f16_row_row_odd": Case(3003, 3001, 2999, "f16", "row", "row", dist="uniform", alpha=0.75,
                            beta=-1.25, has_c=True, act="gelu", seed=71),
    # bf16, column-major A with a padded odd leading dimension, column-major B, bias
    "bf16_col_col_odd": Case(2611, 2603, 2561, "bf16", "col", "col", a_ld=2613, b_ld=2563,
                             bias=True, seed=72),
    "bf16_col_row_odd": Case(2611, 2603, 2561, "bf16", "col", "row", a_ld=2613, b_ld=2605,
                             has_c=True, beta=0.5, seed=73),
    # K not a multiple of 8: both copies are zero-padded to K = 2600
    "bf16_row_col_oddk": Case(2688, 2560, 2599, "bf16", "row", "col", bias=True, act="relu",
                              seed=74),
    # fp8 with row-major B (no 16-byte loader reads a 1-byte operand across K)
    "e4m3_row_row": Case(1536, 1280, 1024, "e4m3", "row", "row", std=1.0, scale_a=0.05,
                         scale_b=0.05, seed=75),
    # fp32 with an odd leading dimension
    "f32_row_row_odd": Case(1031, 1029, 1027, "f32", "row", "row", dist="uniform", a_ld=1029,
                            b_ld=1031, has_c=True, beta=0.5, alpha=1.5, seed=76),
}


def _compare(p, got):
    c = p.case
    if c.M * c.N * c.K <= 1100 ** 3:
        return got.ravel(), p.oracle_full().ravel(), "all outputs"
    return p.oracle_sample(got, seed=9)


@pytest.mark.parametrize("name", list(CASES))
def test_repacked_products_match_oracle(name):
    c = CASES[name]
    p = Prepared(c)
    g, out = p.run()
    info = g.info
    assert info.repack == 1, info.name.decode()
    assert g.workspace_bytes > 0
    got, _ = p.decode_out(out)
    assert np.isfinite(got).all()
    have, want, what = _compare(p, got)
    err = error(c.dtype, have, want)
    print(f"{name}: {info.name.decode()} repack err={err:.3e} on {what}")
    assert err <= TOL[c.dtype], (name, err)


def test_repacked_dyadic_is_bit_exact():
    c = Case(3003, 3001, 2999, "f16", "row", "row", dist="dyadic", alpha=0.75, beta=-1.25,
             has_c=True, bias=True, seed=77)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.repack == 1
    got, _ = p.decode_out(out)
    have, want, what = _compare(p, got)
    ot = OUT_T[c.dtype]
    want_r = oracle.decode(ot, oracle.encode_rne(ot, want))
    assert int((have != want_r).sum()) == 0, what
