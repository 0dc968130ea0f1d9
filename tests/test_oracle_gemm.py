"""Pins for the oracle GEMM against things other than itself: exact rational arithmetic on tiny
shapes, closed forms (identity, permutation, rank-1, alpha = 0), invariants and the normal CDF.

Definition pinned ("CUTLASS", stanleyjacob.dev, Part I and Part II: D = alpha*(A@B) + beta*C,
the epilogue applying alpha/beta, then bias, then activation; Part V "Data types and
quantization": the dequantisation scale is folded into the epilogue).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from hierarchical_tiling_amd import inputs

DT = ["f32", "f16", "bf16", "e4m3"]


def operand(bits, dtype, rows, cols, order, ld=None):
    m = inputs.place(bits, rows, cols, dtype, order, ld)
    return oracle.Operand(m.storage, dtype, m.shape, m.strides), m


def exact_values(bits, dtype):
    return [Fraction(v) for v in oracle.decode(dtype, bits)]


def exact_gemm(a, b, c, bias, M, N, K, alpha, beta, sa, sb, rs=None, cs=None):
    """Exact rational D before activation (a, b, c row-major lists of Fractions; rs, cs optional
    per-row / per-column scale lists)."""
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = sum((a[i * K + k] * b[k * N + j] for k in range(K)), Fraction(0))
            y = Fraction(alpha) * Fraction(sa) * Fraction(sb) * s
            if rs is not None:
                y *= rs[i]
            if cs is not None:
                y *= cs[j]
            if beta != 0:
                y += Fraction(beta) * c[i * N + j]
            if bias is not None:
                y += bias[j]
            row.append(y)
        out.append(row)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    M, N, K = (int(x) for x in rng.integers(1, 7, 3))
    dt = DT[seed % 4]
    dist = "dyadic" if seed % 3 == 0 else "normal"
    a_bits = inputs.quantize(inputs.draw(100 + seed, M * K, dist), dt)
    b_bits = inputs.quantize(inputs.draw(200 + seed, K * N, dist), dt)
    c_dt = "bf16" if dt == "e4m3" else dt
    c_bits = inputs.quantize(inputs.draw(300 + seed, M * N, dist), c_dt)
    bias_bits = inputs.quantize(inputs.draw(400 + seed, N, dist), c_dt)
    A, _ = operand(a_bits, dt, M, K, ["row", "col"][seed % 2], ld=K + 3 if seed % 2 == 0 else M + 1)
    B, _ = operand(b_bits, dt, K, N, ["col", "row"][(seed // 2) % 2])
    C, _ = operand(c_bits, c_dt, M, N, "row", ld=N + 2)
    bias = oracle.Operand(bias_bits, c_dt, (1, N), (N, 1))
    alpha, beta, sa, sb = 1.5, -0.75, 0.5 if dt == "e4m3" else 1.0, 2.0 if dt == "e4m3" else 1.0
    got = oracle.gemm(A, B, C, bias, alpha=alpha, beta=beta, scale_a=sa, scale_b=sb)
    want = exact_gemm(exact_values(a_bits, dt), exact_values(b_bits, dt), exact_values(c_bits, c_dt),
                      exact_values(bias_bits, c_dt), M, N, K, alpha, beta, sa, sb)
    a_abs = [abs(v) for v in exact_values(a_bits, dt)]
    b_abs = [abs(v) for v in exact_values(b_bits, dt)]
    for i in range(M):
        for j in range(N):
            w = want[i][j]
            if dist == "dyadic":
                assert Fraction(got[i, j]) == w  # every partial sum is exact in double
            else:
                mag = sum(a_abs[i * K + k] * b_abs[k * N + j] for k in range(K))
                bound = (K + 4) * 2.0 ** -52 * float(mag * Fraction(alpha) * Fraction(sa) * Fraction(sb) + abs(w)) + 1e-300
                assert abs(got[i, j] - float(w)) <= bound


@pytest.mark.parametrize("seed", range(8))
def test_scale_vectors_match_exact_rationals(seed):
    # D = alpha*sA*sB*row_scale[i]*col_scale[j]*(A@B) + beta*C + bias, each scale an exact float32
    rng = np.random.default_rng(50 + seed)
    M, N, K = (int(x) for x in rng.integers(1, 7, 3))
    dt = DT[seed % 4]
    dist = "dyadic" if seed % 2 == 0 else "normal"
    a_bits = inputs.quantize(inputs.draw(500 + seed, M * K, dist), dt)
    b_bits = inputs.quantize(inputs.draw(600 + seed, K * N, dist), dt)
    c_dt = "bf16" if dt == "e4m3" else dt
    c_bits = inputs.quantize(inputs.draw(700 + seed, M * N, dist), c_dt)
    bias_bits = inputs.quantize(inputs.draw(800 + seed, N, dist), c_dt)
    if dist == "dyadic":   # powers of two: every product stays exact in double
        rs = np.float32(2.0) ** rng.integers(-3, 4, M).astype(np.float32)
        cs = np.float32(2.0) ** rng.integers(-3, 4, N).astype(np.float32)
    else:
        rs = rng.uniform(0.25, 2.0, M).astype(np.float32)
        cs = rng.uniform(-2.0, 2.0, N).astype(np.float32)
    A, _ = operand(a_bits, dt, M, K, "row")
    B, _ = operand(b_bits, dt, K, N, ["col", "row"][seed % 2])
    C, _ = operand(c_bits, c_dt, M, N, "row")
    bias = oracle.Operand(bias_bits, c_dt, (1, N), (N, 1))
    alpha, beta = 0.75, -1.5
    got = oracle.gemm(A, B, C, bias, alpha=alpha, beta=beta, row_scale=rs, col_scale=cs)
    ex_rs = [Fraction(float(v)) for v in rs]
    ex_cs = [Fraction(float(v)) for v in cs]
    want = exact_gemm(exact_values(a_bits, dt), exact_values(b_bits, dt), exact_values(c_bits, c_dt),
                      exact_values(bias_bits, c_dt), M, N, K, alpha, beta, 1.0, 1.0, ex_rs, ex_cs)
    a_abs = [abs(v) for v in exact_values(a_bits, dt)]
    b_abs = [abs(v) for v in exact_values(b_bits, dt)]
    for i in range(M):
        for j in range(N):
            w = want[i][j]
            if dist == "dyadic":
                assert Fraction(got[i, j]) == w
            else:
                mag = sum(a_abs[i * K + k] * b_abs[k * N + j] for k in range(K))
                scale = abs(Fraction(alpha) * ex_rs[i] * ex_cs[j])
                bound = (K + 6) * 2.0 ** -52 * float(mag * scale + abs(w)) + 1e-300
                assert abs(got[i, j] - float(w)) <= bound


def test_scale_vectors_are_row_and_column_broadcasts():
    # with power-of-two scales the fused result equals diag(rs) @ D @ diag(cs) bit for bit
    M, N, K = 9, 7, 13
    A, _ = operand(inputs.quantize(inputs.draw(31, M * K), "bf16"), "bf16", M, K, "row")
    B, _ = operand(inputs.quantize(inputs.draw(32, K * N), "bf16"), "bf16", K, N, "col")
    rs = np.float32(2.0) ** np.arange(-4, M - 4, dtype=np.float32)
    cs = np.float32(2.0) ** -np.arange(N, dtype=np.float32)
    plain = oracle.gemm(A, B)
    fused = oracle.gemm(A, B, row_scale=rs, col_scale=cs)
    np.testing.assert_array_equal(fused, rs[:, None].astype(np.float64) * plain * cs[None, :])
    only_c = oracle.gemm(A, B, col_scale=cs)
    np.testing.assert_array_equal(only_c, plain * cs[None, :])
    with pytest.raises(ValueError):
        oracle.gemm(A, B, row_scale=rs[:-1])


def test_silu_odd_part_and_tanh_form():
    # SiLU(x) = x * sigmoid(x).  Since sigmoid(x) + sigmoid(-x) = 1, SiLU(x) - SiLU(-x) = x; and
    # sigmoid(x) = (1 + tanh(x / 2)) / 2 gives a second closed form through the library tanh.
    x = np.array([-30.0, -4.0, -1.0, -0.25, 0.0, 0.25, 1.0, 4.0, 30.0])
    A, _ = operand(inputs.quantize(np.ones(1), "f32"), "f32", 1, 1, "row")
    B, _ = operand(inputs.quantize(x, "f32"), "f32", 1, x.size, "row")
    Bn, _ = operand(inputs.quantize(-x, "f32"), "f32", 1, x.size, "row")
    silu = oracle.gemm(A, B, act="silu")[0]
    sneg = oracle.gemm(A, Bn, act="silu")[0]
    np.testing.assert_allclose(silu - sneg, x, rtol=0, atol=4e-15)
    # (the tanh form cancels for very negative x, so its absolute error, not its relative one,
    # stays near 1e-16 there)
    tanh_form = np.array([v * (1.0 + math.tanh(v / 2.0)) / 2.0 for v in x])
    np.testing.assert_allclose(silu, tanh_form, rtol=1e-14, atol=1e-14)
    assert silu[4] == 0.0
    assert silu[0] < 0 and abs(silu[0]) < 1e-11 and silu[-1] == pytest.approx(30.0, rel=1e-12)


@pytest.mark.parametrize("dt", DT)
def test_identity_times_b(dt):
    n, N = 7, 5
    eye = inputs.quantize(np.eye(n).ravel(), dt)
    b_bits = inputs.quantize(inputs.draw(5, n * N, "normal"), dt)
    A, _ = operand(eye, dt, n, n, "row")
    B, _ = operand(b_bits, dt, n, N, "col")
    got = oracle.gemm(A, B, alpha=2.0)
    np.testing.assert_array_equal(got, 2.0 * oracle.decode(dt, b_bits).reshape(n, N))


def test_permutation_reorders_rows():
    n, N = 9, 4
    perm = np.random.default_rng(3).permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1.0
    b_bits = inputs.quantize(inputs.draw(6, n * N, "uniform"), "bf16")
    A, _ = operand(inputs.quantize(P.ravel(), "bf16"), "bf16", n, n, "col")
    B, _ = operand(b_bits, "bf16", n, N, "row")
    got = oracle.gemm(A, B)
    bvals = oracle.decode("bf16", b_bits).reshape(n, N)
    np.testing.assert_array_equal(got, bvals[perm])


def test_rank_one_closed_form():
    M, N, K = 5, 6, 33
    u = inputs.quantize(inputs.draw(7, M, "dyadic"), "f16")
    v = inputs.quantize(inputs.draw(8, N, "dyadic"), "f16")
    uv, vv = oracle.decode("f16", u), oracle.decode("f16", v)
    A, _ = operand(np.repeat(u, K), "f16", M, K, "row")          # A = u 1^T
    B, _ = operand(np.tile(v, K), "f16", K, N, "row")            # B = 1 v^T
    got = oracle.gemm(A, B, alpha=0.5)
    np.testing.assert_array_equal(got, 0.5 * K * np.outer(uv, vv))


def test_alpha_zero_passes_beta_c_through():
    M, N, K = 4, 3, 5
    A, _ = operand(inputs.quantize(inputs.draw(1, M * K), "f32"), "f32", M, K, "row")
    B, _ = operand(inputs.quantize(inputs.draw(2, K * N), "f32"), "f32", K, N, "row")
    c_bits = inputs.quantize(inputs.draw(3, M * N), "f32")
    C, _ = operand(c_bits, "f32", M, N, "row")
    got = oracle.gemm(A, B, C, alpha=0.0, beta=-1.25)
    np.testing.assert_array_equal(got, -1.25 * oracle.decode("f32", c_bits).reshape(M, N))


def test_beta_zero_never_reads_c():
    M, N, K = 3, 4, 2
    A, _ = operand(inputs.quantize(inputs.draw(1, M * K), "f32"), "f32", M, K, "row")
    B, _ = operand(inputs.quantize(inputs.draw(2, K * N), "f32"), "f32", K, N, "row")
    C, _ = operand(inputs.quantize(np.full(M * N, np.nan), "f32"), "f32", M, N, "row")
    assert np.isfinite(oracle.gemm(A, B, C, beta=0.0)).all()
    assert np.isfinite(oracle.gemm(A, B, None, beta=0.0)).all()
    with pytest.raises(ValueError):
        oracle.gemm(A, B, None, beta=1.0)  # beta != 0 needs C


def test_bias_is_per_column():
    M, N, K = 3, 5, 2
    A, _ = operand(inputs.quantize(np.zeros(M * K), "bf16"), "bf16", M, K, "row")
    B, _ = operand(inputs.quantize(np.zeros(K * N), "bf16"), "bf16", K, N, "col")
    bias_bits = inputs.quantize(np.arange(N, dtype=float), "bf16")
    got = oracle.gemm(A, B, None, oracle.Operand(bias_bits, "bf16", (1, N), (N, 1)))
    np.testing.assert_array_equal(got, np.tile(np.arange(N, dtype=float), (M, 1)))


def test_power_of_two_scaling_is_exact():
    M, N, K = 6, 7, 40
    a = inputs.draw(11, M * K, "normal")
    b_bits = inputs.quantize(inputs.draw(12, K * N, "normal"), "bf16")
    a1 = inputs.quantize(a, "bf16")
    a2 = inputs.quantize(2.0 * a, "bf16")
    B, _ = operand(b_bits, "bf16", K, N, "col")
    d1 = oracle.gemm(operand(a1, "bf16", M, K, "row")[0], B)
    d2 = oracle.gemm(operand(a2, "bf16", M, K, "row")[0], B)
    np.testing.assert_array_equal(d2, 2.0 * d1)


def test_activations():
    x = np.array([-3.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0, 10.0])
    M, N = 1, x.size
    A, _ = operand(inputs.quantize(np.ones(1), "f32"), "f32", 1, 1, "row")
    B, _ = operand(inputs.quantize(x, "f32"), "f32", 1, N, "row")
    relu = oracle.gemm(A, B, act="relu")[0]
    np.testing.assert_array_equal(relu, np.maximum(x, 0.0))
    gelu = oracle.gemm(A, B, act="gelu")[0]
    # GELU(x) = x * Phi(x); Phi(1) = 0.8413447460685429 (standard normal CDF table value)
    assert abs(gelu[5] - 0.8413447460685429) < 1e-15
    # x*Phi(x) - (-x)*Phi(-x) = x for every x, since Phi(x) + Phi(-x) = 1
    Bn, _ = operand(inputs.quantize(-x, "f32"), "f32", 1, N, "row")
    gneg = oracle.gemm(A, Bn, act="gelu")[0]
    np.testing.assert_allclose(gelu - gneg, x, rtol=0, atol=1e-15)
    assert gelu[3] == 0.0 and gelu[7] == pytest.approx(10.0, abs=1e-20)


def test_elements_equal_full_result_and_threads_do_not_change_bits():
    M, N, K = 37, 29, 51
    A, _ = operand(inputs.quantize(inputs.draw(21, M * K), "f16"), "f16", M, K, "col", ld=40)
    B, _ = operand(inputs.quantize(inputs.draw(22, K * N), "f16"), "f16", K, N, "row", ld=31)
    C, _ = operand(inputs.quantize(inputs.draw(23, M * N), "f16"), "f16", M, N, "row")
    kw = dict(alpha=0.75, beta=-1.25, act="gelu")
    full1 = oracle.gemm(A, B, C, threads=1, **kw)
    full8 = oracle.gemm(A, B, C, threads=8, **kw)
    np.testing.assert_array_equal(full1, full8)
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, M, 300), rng.integers(0, N, 300)
    el = oracle.gemm_elems(A, B, rows, cols, C, threads=5, **kw)
    np.testing.assert_array_equal(el, full1[rows, cols])


def test_padding_between_rows_is_ignored():
    M, N, K = 4, 4, 4
    vals = inputs.quantize(inputs.draw(31, M * K, "dyadic"), "f32")
    Ap = inputs.place(vals, M, K, "f32", "row", ld=9, fill=0x7FC00000)  # NaN in the padding
    A = oracle.Operand(Ap.storage, "f32", Ap.shape, Ap.strides)
    B, _ = operand(inputs.quantize(np.eye(4).ravel(), "f32"), "f32", K, N, "row")
    np.testing.assert_array_equal(oracle.gemm(A, B), oracle.decode("f32", vals).reshape(M, K))


def test_empty_shapes():
    A = oracle.Operand(np.zeros(0, np.uint16), "bf16", (0, 5), (5, 1))
    B = oracle.Operand(np.zeros(25, np.uint16), "bf16", (5, 5), (5, 1))
    assert oracle.gemm(A, B).shape == (0, 5)
    A0 = oracle.Operand(np.zeros(0, np.uint16), "bf16", (3, 0), (1, 1))
    B0 = oracle.Operand(np.zeros(0, np.uint16), "bf16", (0, 2), (1, 1))
    np.testing.assert_array_equal(oracle.gemm(A0, B0), np.zeros((3, 2)))   # K = 0: empty sum


# ---- reductions of the stored output (the next layer's normalisation inputs) ----------------
# Reading of "CUTLASS", Part IV Stage 5 (a fused reduction for the next layer's norm): the sum of
# squares of each row and the sum of each column of D as stored, i.e. rounded to the output type.

def test_reductions_round_before_summing_hand_values():
    # 1 + 2^-9 lies below the bf16 midpoint of 1 and 1 + 2^-7 and rounds to 1; 1 + 2^-8 is that
    # midpoint and rounds to the even neighbour 1; both are exact in fp16 (10 stored bits).
    D = np.array([[1 + 2.0 ** -9, 3.0, -0.5], [2.0, 1 + 2.0 ** -8, 0.25]])
    assert oracle.row_sumsq(D, "bf16").tolist() == [1 + 9 + 0.25, 4 + 1 + 0.0625]
    assert oracle.col_sum(D, "bf16").tolist() == [3.0, 4.0, -0.25]
    f16 = oracle.row_sumsq(D, "f16")
    x, y = Fraction(1) + Fraction(1, 512), Fraction(1) + Fraction(1, 256)
    assert Fraction(f16[0]) == x * x + 9 + Fraction(1, 4)
    assert Fraction(f16[1]) == 4 + y * y + Fraction(1, 16)
    assert oracle.col_sum(D, "f16").tolist() == [3 + 2.0 ** -9, 4 + 2.0 ** -8, -0.25]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_reductions_of_a_constant_matrix(dt):
    # every stored value is r = round(1/3): row sums of squares are N r^2, column sums M r
    M, N = 7, 5
    r = Fraction(float(oracle.decode(dt, oracle.encode_rne(dt, np.array([1 / 3])))[0]))
    D = np.full((M, N), 1 / 3)
    assert all(Fraction(v) == N * r * r for v in oracle.row_sumsq(D, dt))
    assert all(Fraction(v) == M * r for v in oracle.col_sum(D, dt))


def test_reductions_of_identity_times_b_are_those_of_b():
    # D = I @ B with B already in the output type: every stored D value is B's, so the reductions
    # are B's own row sums of squares and column sums, computed here with exact rationals
    K, N = 6, 9
    b_bits = inputs.quantize(inputs.draw(77, K * N, "normal"), "bf16")
    eye = inputs.quantize(np.eye(K).ravel(), "bf16")
    A, _ = operand(eye, "bf16", K, K, "row")
    B, _ = operand(b_bits, "bf16", K, N, "col")
    D = oracle.gemm(A, B)
    b = exact_values(b_bits, "bf16")
    for i, v in enumerate(oracle.row_sumsq(D, "bf16")):
        assert Fraction(v) == sum(b[i * N + j] ** 2 for j in range(N))
    for j, v in enumerate(oracle.col_sum(D, "bf16")):
        assert Fraction(v) == sum(b[i * N + j] for i in range(K))


def test_reductions_of_empty_shapes():
    assert oracle.row_sumsq(np.zeros((3, 0)), "bf16").tolist() == [0.0, 0.0, 0.0]
    assert oracle.col_sum(np.zeros((0, 2)), "bf16").tolist() == [0.0, 0.0]
