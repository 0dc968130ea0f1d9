"""GPU parity on seeded random problems through the library's own kernel choice (160 small, 16 mid-size).

Each case draws a shape (small to a few tiles, with ragged tails in M, N and K), operand type,
layouts, padded leading dimensions, output order and epilogue (alpha, beta with C, bias,
activation, fp8 scales), runs it through the C ABI and compares with the CPU oracle.  Dyadic cases
(multiples of 1/4: every fp32 partial sum exact) must match bit for bit; the others must meet the
type's tolerance (fp32 relative Frobenius 1e-5, bf16/fp16 max-abs-relative 1e-2, fp8 3e-2).
"""
import random

import numpy as np
import pytest

import oracle
from tests.gemm_util import OUT_T, TOL, Case, Prepared, error

pytestmark = pytest.mark.gpu

N_CASES = 160


def draw(i):
    rng = random.Random(9000 + i)
    dtype = rng.choice(["f32", "f16", "bf16", "bf16", "e4m3"])
    # about two thirds of the sizes and pads keep 16-byte rows (the vector and DMA loaders), the
    # rest are odd (the realigned and element loaders)
    def dim():
        d = rng.choice([rng.randint(1, 40), rng.randint(41, 300), 256 * rng.randint(1, 2),
                        rng.randint(257, 600)])
        return max(16, d - d % 16) if rng.random() < 0.65 else d
    M, N, K = dim(), dim(), dim()
    a_order, b_order = rng.choice(["row", "col"]), rng.choice(["row", "col"])
    pad = lambda: rng.choice([0, 0, 0, 16, 64, 13])
    a_ld = (K if a_order == "row" else M) + pad()
    b_ld = (N if b_order == "row" else K) + pad()
    d_order = rng.choice(["row", "row", "col"])
    has_c = rng.random() < 0.4
    dyadic = rng.random() < 0.3
    c = Case(M=M, N=N, K=K, dtype=dtype, a_order=a_order, b_order=b_order,
             dist="dyadic" if dyadic else ("uniform" if dtype == "f32" else "normal"),
             alpha=rng.choice([1.0, 0.5, 2.0] if dyadic else [1.0, 0.75, -1.5]),
             beta=rng.choice([0.5, -2.0]) if has_c else 0.0, has_c=has_c,
             bias=rng.random() < 0.5,
             act="none" if dyadic else rng.choice(["none", "relu", "gelu", "silu"]),
             scale_a=rng.choice([0.5, 1.0, 2.0]) if dtype == "e4m3" else 1.0,
             scale_b=rng.choice([0.25, 1.0]) if dtype == "e4m3" else 1.0,
             a_ld=a_ld, b_ld=b_ld, d_order=d_order, seed=9000 + i)
    return c, dyadic


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem_matches_oracle(i):
    c, dyadic = draw(i)
    p = Prepared(c)
    g, out = p.run()
    got, bits = p.decode_out(out)
    want = p.oracle_full()
    name = g.info.name.decode()
    print(f"case {i}: {c.dtype} {c.M}x{c.N}x{c.K} {c.a_order}/{c.b_order} ld=({c.a_ld},{c.b_ld}) "
          f"d={c.d_order} C={c.has_c} bias={c.bias} act={c.act} -> {name}")
    if dyadic:
        exp = oracle.encode_rne(OUT_T[c.dtype], want)
        assert int((bits != exp).sum()) == 0, name
    else:
        assert np.isfinite(got).all()
        assert error(c.dtype, got, want) <= TOL[c.dtype], name


# Mid-size problems (one-round ring choices, K splits, split tails), checked on sampled outputs:
# whole first/last rows and columns plus random elements.
N_MID = 16


def draw_mid(i):
    rng = random.Random(9500 + i)
    dtype = rng.choice(["bf16", "bf16", "f16", "e4m3"])
    M, N = rng.randint(1100, 4400), rng.randint(1100, 4400)
    if rng.random() < 0.6:
        M, N = M - M % 16, N - N % 16
    K = rng.choice([512, 1024, 2048, 4096, 8192]) + rng.choice([0, 0, 64, 48])
    dyadic = rng.random() < 0.5
    c = Case(M=M, N=N, K=K, dtype=dtype, a_order="row", b_order="col",
             dist="dyadic" if dyadic else "normal", alpha=1.0 if dyadic else 0.75,
             beta=0.5 if rng.random() < 0.4 else 0.0, bias=rng.random() < 0.5,
             act="none" if dyadic else rng.choice(["none", "gelu", "silu"]),
             scale_a=0.5 if dtype == "e4m3" else 1.0, scale_b=0.5 if dtype == "e4m3" else 1.0,
             seed=9500 + i)
    c.has_c = c.beta != 0.0
    return c, dyadic


@pytest.mark.parametrize("i", range(N_MID))
def test_random_mid_size_problem_matches_oracle(i):
    from tests.gemm_util import sample_indices
    c, dyadic = draw_mid(i)
    p = Prepared(c)
    g, out = p.run()
    got, bits = p.decode_out(out)
    rows, cols = sample_indices(c.M, c.N, seed=i)
    want = p.oracle_elems(rows, cols)
    inf = g.info
    print(f"mid {i}: {c.dtype} {c.M}x{c.N}x{c.K} C={c.has_c} bias={c.bias} act={c.act} -> "
          f"{inf.name.decode()} split={inf.split_k} tail={inf.tail_tiles}x{inf.tail_split}")
    if dyadic:
        assert int((bits[rows, cols] != oracle.encode_rne(OUT_T[c.dtype], want)).sum()) == 0
    else:
        assert np.isfinite(got).all()
        assert error(c.dtype, got[rows, cols], want) <= TOL[c.dtype]
