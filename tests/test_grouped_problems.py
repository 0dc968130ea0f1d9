"""Grouped GEMM of independent problems ("CUTLASS", Part III: a grouped GEMM runs many problems of
irregular shapes in one launch): every problem has its own M, N, K, pointers and leading
dimensions, and each is compared with the oracle on its own.  Output buffers start as a NaN
sentinel, so a write outside a problem's M x N (into the padding of its leading dimension or past
its end) is caught."""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_tiling_amd import htgemm as H
from hierarchical_tiling_amd import inputs

from gemm_util import OUT_T, THREADS, TOL, error, op

pytestmark = pytest.mark.gpu

RING = "bf16_ak_bk_256x256x64_w2x4_m16_ring"

# (M, N, K) per problem, plus the padding of each leading dimension (elements)
CASES = {
    # the split ring forced: an empty problem, a one-row problem, K = 0, tile-edge shapes
    "bf16_ring_mixed": dict(dtype="bf16", shapes=[(300, 264, 320), (0, 100, 64), (1, 520, 128),
                                                  (517, 130, 64), (64, 72, 0), (256, 256, 512)],
                            pad=8, bias=True, act="gelu", force=RING),
    # column-major A, row-major B, C with beta, column-major D: the library's choice
    "f16_mn_major_c": dict(dtype="f16", shapes=[(96, 200, 64), (136, 64, 136), (40, 8, 24)],
                           a_order="col", b_order="row", d_order="col", pad=16, has_c=True,
                           beta=-0.5, alpha=1.5),
    # one leading dimension off the 16-byte grid: every problem runs on the narrow loaders
    "bf16_odd_ld": dict(dtype="bf16", shapes=[(128, 136, 96), (70, 33, 40)], pad=8, odd_ld=1,
                        bias=True),
    "e4m3_scales": dict(dtype="e4m3", shapes=[(260, 300, 256), (16, 520, 512), (64, 64, 128)],
                        pad=16, scale_a=0.5, scale_b=0.25, bias=True, act="silu"),
    # 40 small problems of random shapes (some empty), fp32 with C
    "f32_forty": dict(dtype="f32", shapes="random40", pad=4, has_c=True, beta=1.0, alpha=0.5,
                      dist="uniform"),
    # problems of many tiles each: the library's choice for a typical 1024 x 768 x 512 problem
    "bf16_large": dict(dtype="bf16", shapes=[(1024, 768, 512), (256, 2048, 1024), (1536, 512, 256)],
                       pad=0, bias=True, typical=(1024, 768, 512)),
}


def _shapes(spec, seed):
    if spec != "random40":
        return spec
    rng = np.random.default_rng(seed)
    return [tuple(int(v) for v in rng.integers(0, 150, 3)) for _ in range(40)]


def _table():
    return [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_problems_match_oracle_each(name):
    kw = dict(CASES[name])
    dt = kw["dtype"]
    ot = OUT_T[dt]
    seed = 700 + list(CASES).index(name) * 50
    shapes = _shapes(kw["shapes"], seed)
    pad, odd = kw.get("pad", 0), kw.get("odd_ld", 0)
    a_order, b_order = kw.get("a_order", "row"), kw.get("b_order", "col")
    d_order = kw.get("d_order", "row")
    has_c, beta, alpha = kw.get("has_c", False), kw.get("beta", 0.0), kw.get("alpha", 1.0)
    sa, sb = kw.get("scale_a", 1.0), kw.get("scale_b", 1.0)
    dist = kw.get("dist", "normal")
    sentinel = oracle.encode_rne(ot, np.array([np.nan]))[0]
    keep = []          # device tensors alive until the launch has finished
    probs, host = [], []
    for i, (M, N, K) in enumerate(shapes):
        s = seed + 7 * i
        ex = dict(std=max(K, 1) ** -0.5) if dist == "normal" else {}
        a_ld = (K if a_order == "row" else M) + pad + (odd if i == 0 else 0)
        b_ld = (K if b_order == "col" else N) + pad
        A = inputs.matrix(s + 1, M, K, dt, dist, order=a_order, ld=max(a_ld, 1), **ex)
        B = inputs.matrix(s + 2, K, N, dt, dist, order=b_order, ld=max(b_ld, 1), **ex)
        C = inputs.matrix(s + 3, M, N, ot, "uniform", order="row", ld=N + pad) if has_c else None
        bias = inputs.vector(s + 4, N, ot, "normal", std=0.1) if kw.get("bias") else None
        d_strides, d_len = inputs.layout_strides(M, N, d_order, (N if d_order == "row" else M) + pad)
        tail = 29
        d_host = np.full(d_len + tail, sentinel, dtype=inputs.STORAGE[ot])
        dev = lambda m: inputs.to_device(m) if m is not None and m.storage.size else None
        dA, dB, dC, dbias = dev(A), dev(B), dev(C), dev(bias)
        dD = torch.from_numpy(d_host).to("cuda")
        keep += [dA, dB, dC, dbias, dD]
        addr = lambda t: t.data_ptr() if t is not None else None
        probs.append(dict(M=M, N=N, K=K, A=addr(dA), B=addr(dB), C=addr(dC), D=dD.data_ptr(),
                          bias=addr(dbias),
                          lda=A.strides[0] if a_order == "row" else A.strides[1],
                          ldb=B.strides[1] if b_order == "col" else B.strides[0],
                          ldc=C.strides[0] if C is not None else 0,
                          ldd=d_strides[0] if d_order == "row" else d_strides[1]))
        host.append((A, B, C, bias, d_strides, d_len, dD))
    M0, N0, K0 = kw.get("typical", max(shapes, key=lambda t: t[0] * t[1] * max(t[2], 1)))
    a_str = (K0 + pad, 1) if a_order == "row" else (1, M0 + pad)
    b_str = (1, K0 + pad) if b_order == "col" else (N0 + pad, 1)
    d_str = (N0 + pad, 1) if d_order == "row" else (1, M0 + pad)
    force = _table().index(kw["force"]) if "force" in kw else -1
    desc = H.make_desc(M0, N0, K0, dt, a_str, b_str, d_str,
                       c_strides=(N0 + pad, 1) if has_c else None, has_bias=kw.get("bias", False),
                       act=kw.get("act", "none"), force_config=force, batch=len(shapes),
                       grouped=True)
    g = H.Gemm(desc)
    # the problem table lives in the workspace, which starts as garbage
    ws = torch.full((g.workspace_bytes // 4,), -1, dtype=torch.int32, device="cuda")
    H.gemm_run_problems(g.handle, probs, alpha, beta, sa, sb,
                        torch.cuda.current_stream().cuda_stream, ws.data_ptr())
    torch.cuda.synchronize()
    name_k = g.info.name.decode()
    for i, ((M, N, K), (A, B, C, bias, d_strides, d_len, dD)) in enumerate(zip(shapes, host)):
        bits = dD.cpu().numpy().view(inputs.STORAGE[ot])
        assert (bits[d_len:] == sentinel).all(), f"problem {i} wrote past its D"
        if M == 0 or N == 0:
            assert (bits == sentinel).all()
            continue
        r = np.arange(M)[:, None] * d_strides[0] + np.arange(N)[None, :] * d_strides[1]
        inside = np.zeros(bits.size, dtype=bool)
        inside[r.ravel()] = True
        assert (bits[~inside] == sentinel).all(), f"problem {i} wrote into its padding"
        got = oracle.decode(ot, bits[r])
        want = oracle.gemm(op(A), op(B), op(C) if C is not None else None,
                           op(bias) if bias is not None else None, alpha=alpha, beta=beta,
                           scale_a=sa, scale_b=sb, act=kw.get("act", "none"), threads=THREADS)
        err = error(dt, got, want)
        if len(shapes) <= 8:
            print(f"{name}[{i}] {M}x{N}x{K}: {name_k} err={err:.3e}")
        assert err <= TOL[dt], (name, i, (M, N, K), err)
    if "force" in kw:
        assert name_k == kw["force"]


def test_grouped_problems_equal_single_runs_bit_for_bit():
    """The same tile kernel on the same problem gives the same bits whether the problem runs
    alone or inside a group (the per-element sums do not depend on the launch)."""
    dt, ot = "bf16", "bf16"
    shapes = [(320, 280, 192), (96, 512, 64), (257, 255, 128)]
    force = _table().index(RING)
    outs_g, outs_1, keep, probs = [], [], [], []
    for i, (M, N, K) in enumerate(shapes):
        A = inputs.matrix(900 + i, M, K, dt, "normal", order="row", std=K ** -0.5)
        B = inputs.matrix(950 + i, K, N, dt, "normal", order="col", std=K ** -0.5)
        bias = inputs.vector(990 + i, N, ot, "normal", std=0.1)
        dA, dB, dbias = inputs.to_device(A), inputs.to_device(B), inputs.to_device(bias)
        dDg = torch.zeros(M * N * 2, dtype=torch.uint8, device="cuda")
        dD1 = torch.zeros(M * N * 2, dtype=torch.uint8, device="cuda")
        keep += [dA, dB, dbias]
        outs_g.append(dDg)
        outs_1.append(dD1)
        probs.append(dict(M=M, N=N, K=K, A=dA.data_ptr(), B=dB.data_ptr(), D=dDg.data_ptr(),
                          bias=dbias.data_ptr(), lda=K, ldb=K, ldd=N))
        g1 = H.Gemm(H.make_desc(M, N, K, dt, (K, 1), (1, K), (N, 1), has_bias=True, act="gelu",
                                force_config=force, split_k=1))
        g1.run(dA, dB, None, dD1, dbias)
    g = H.Gemm(H.make_desc(320, 280, 192, dt, (192, 1), (1, 192), (280, 1), has_bias=True,
                           act="gelu", force_config=force, batch=len(shapes), grouped=True))
    ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda")
    H.gemm_run_problems(g.handle, probs, 1.0, 0.0, workspace=ws.data_ptr())
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(outs_g[i], outs_1[i]), i


def test_grouped_problems_run_twice_with_fewer_problems():
    """A handle runs any count up to its batch; a second, smaller call reuses the workspace."""
    dt = "f16"
    force = -1
    shapes = [(64, 64, 64), (128, 96, 32), (33, 17, 48)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A = inputs.matrix(1100 + i, M, K, dt, "normal", order="row", std=K ** -0.5)
        B = inputs.matrix(1150 + i, K, N, dt, "normal", order="col", std=K ** -0.5)
        data.append((A, B, inputs.to_device(A), inputs.to_device(B)))
    g = H.Gemm(H.make_desc(64, 64, 64, dt, (64, 1), (1, 64), (64, 1), force_config=force,
                           batch=len(shapes), grouped=True))
    ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda")
    for count in (3, 2):
        outs, probs = [], []
        for i in range(count):
            M, N, K = shapes[i]
            A, B, dA, dB = data[i]
            dD = torch.zeros(M * N * 2, dtype=torch.uint8, device="cuda")
            outs.append(dD)
            probs.append(dict(M=M, N=N, K=K, A=dA.data_ptr(), B=dB.data_ptr(), D=dD.data_ptr(),
                              lda=K, ldb=K, ldd=N))
        H.gemm_run_problems(g.handle, probs, 1.0, 0.0, workspace=ws.data_ptr())
        torch.cuda.synchronize()
        for i in range(count):
            M, N, K = shapes[i]
            A, B, _, _ = data[i]
            got = oracle.decode("f16", outs[i].cpu().numpy().view(np.uint16)).reshape(M, N)
            want = oracle.gemm(op(A), op(B), None, None, threads=THREADS)
            assert error(dt, got, want) <= TOL[dt], (count, i)


def test_grouped_problems_many_small():
    """1,500 problems of 0..40 rows and columns: the binary search over the problems' first tiles
    and the table copy at a size where most workgroups belong to problems deep in the table."""
    rng = np.random.default_rng(77)
    G = 1500
    shapes = [(int(m), int(n), 32) for m, n in zip(rng.integers(0, 41, G), rng.integers(0, 41, G))]
    dt, ot = "bf16", "bf16"
    A_all = inputs.matrix(7000, sum(m for m, _, _ in shapes) + 1, 32, dt, "dyadic", order="row")
    B_all = inputs.matrix(7001, 32, 40 * G, dt, "dyadic", order="col")
    dA, dB = inputs.to_device(A_all), inputs.to_device(B_all)
    D = torch.zeros(sum(m * n for m, n, _ in shapes) + 8, dtype=torch.int16, device="cuda")
    probs, where, r0, d0 = [], [], 0, 0
    for e, (m, n, k) in enumerate(shapes):
        probs.append(dict(M=m, N=n, K=k, A=dA.data_ptr() + r0 * 32 * 2,
                          B=dB.data_ptr() + e * 40 * 32 * 2, D=D.data_ptr() + d0 * 2,
                          lda=32, ldb=32, ldd=max(n, 1)))
        where.append((r0, e * 40, d0))
        r0 += m
        d0 += m * n
    g = H.Gemm(H.make_desc(32, 32, 32, dt, (32, 1), (1, 32), (32, 1), batch=G, grouped=True))
    ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda")
    H.gemm_run_problems(g.handle, probs, 1.0, 0.0, workspace=ws.data_ptr())
    torch.cuda.synchronize()
    bits = D.cpu().numpy().view(np.uint16)
    bad = 0
    for (m, n, k), (ra, cb, dd) in zip(shapes, where):
        if m == 0 or n == 0:
            continue
        A_e = oracle.Operand(A_all.storage[ra * 32:], dt, (m, 32), (32, 1))
        B_e = oracle.Operand(B_all.storage[cb * 32:], dt, (32, n), (1, 32))
        want = oracle.gemm(A_e, B_e, None, None, threads=1)
        # dyadic inputs: every sum is exact, so the stored bits are unique
        bad += int((bits[dd:dd + m * n] != oracle.encode_rne(ot, want).ravel()).sum())
    assert bad == 0
