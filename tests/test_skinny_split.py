"""GPU parity of the streaming kernel for M <= 16 when its column blocks do not fill the GPU and
K is cut into slices (fp32 planes summed in fixed order by the split-K sum kernel): the
profiler-lab shape of the pages (16 x 16 x 32768, small M and N, long K) and narrow ragged
variants, against the oracle; dyadic inputs bit for bit."""
import numpy as np
import pytest

import oracle
from hierarchical_tiling_amd import htgemm as H
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error

pytestmark = pytest.mark.gpu

CASES = {
    # small M and N, long K ("CUTLASS", Part VII: the profiler lab's split-K shape)
    "bf16_16x16x32768": Case(16, 16, 32768, "bf16", seed=700),
    # ragged M, N and K (a K tail inside the last block of the last slice), C and bias
    "f16_13x40x20000": Case(13, 40, 20000, "f16", has_c=True, beta=-0.5, alpha=0.75, bias=True,
                            act="gelu", seed=701),
    "e4m3_8x600x16384": Case(8, 600, 16384, "e4m3", std=1.0, scale_a=0.5, scale_b=0.25, seed=702),
    # scale vectors through the sum kernel's epilogue
    "bf16_16x256x8192_scales": Case(16, 256, 8192, "bf16", row_scale=True, col_scale=True,
                                    act="silu", seed=703),
}


@pytest.mark.parametrize("name", list(CASES))
def test_split_skinny_matches_oracle(name):
    c = CASES[name]
    p = Prepared(c)
    g, out = p.run()
    info = g.info
    assert "skinny_dma" in info.name.decode() and info.split_k > 1, (info.name, info.split_k)
    got, _ = p.decode_out(out)
    err = error(c.dtype, got, p.oracle_full())
    print(f"{name}: {info.name.decode()} split {info.split_k} err={err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[c.dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_split_skinny_dyadic_bit_exact(dtype):
    c = Case(11, 72, 16384, dtype, dist="dyadic", alpha=2.0, beta=0.5, has_c=True, bias=True,
             seed=710, scale_a=0.5 if dtype == "e4m3" else 1.0,
             scale_b=2.0 if dtype == "e4m3" else 1.0)
    p = Prepared(c)
    g, out = p.run()
    assert g.info.split_k > 1
    _, bits = p.decode_out(out)
    want = oracle.encode_rne(OUT_T[dtype], p.oracle_full())
    assert int((bits != want).sum()) == 0
