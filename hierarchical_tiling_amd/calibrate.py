"""Measures the tile table's cost model on the GPU and writes it as C++ source.

    python -m hierarchical_tiling_amd.calibrate --out FILE [--only REGEX] [--reps R] [--passes P]
    python -m hierarchical_tiling_amd.calibrate --check --out FILE

The library chooses a kernel by predicting each fitting entry's time on the problem ("CUTLASS",
stanleyjacob.dev, Part IX: the best tile depends on the shape, so the library measures its
kernels rather than guessing).  The prediction rests on two measured numbers per entry and per
load (workgroups per compute unit: 1/4, 1/2, 3/4, then n = 1..8): a fixed cost f and a cost per
k-tile c, in microseconds, so that a launch of 256 * load workgroups of kt k-tiles each takes
f + kt * c.  Between the loads below one the library interpolates; a load above 8 is taken as
whole groups of 8 plus the rest.

For each entry (the streaming kernels for M <= 16 excepted: they are chosen by their shape) this
script forces the entry on products with exactly 256 * load tiles, at two depths, and fits the
two numbers to the median of several passes over the table; it also measures the extra time of
a partial last k-tile, of partial last tile rows and columns and of output rows off 16 bytes.
Entries that load through realigned
or element-wise loaders are measured with odd leading dimensions (the case they serve); the
others with aligned, packed operands.  Operands are normal random values.  It then measures the
split-K second kernel, whose cost is modelled as g0 + g1 * bytes (its fp32 partial planes, written
and read, plus the output), and the copies into aligned K-major buffers (h0 + h1 * bytes, read and
written) from products that the library runs on such copies, and Stream-K launches (s0 + s1 times
the entry's time for 256 workgroups of one share) against the prediction for their whole tiles.

The output is the source of the library's cost table (csrc/cost_table.cpp); rebuild after
replacing it.  With --check the script instead times the library's automatic choice against every
fitting entry on a fixed set of products and reports how far the choice is from the best.
"""
from __future__ import annotations

import argparse
import re
import sys
import time

KT = (16, 64)          # the two depths, in k-tiles
LOADS = (0.25, 0.5, 0.75, 1, 2, 3, 4, 5, 6, 7, 8)   # workgroups per compute unit
ONE = LOADS.index(1)                               # index of the load 1
CUS = 256


def parse_name(name):
    """(dtype, a_kmajor, b_kmajor, kind) of an entry from its name, where kind is vec, narrow,
    realign, dma, ring or skinny."""
    parts = name.split("_")
    dtype, a, b = parts[0], parts[1], parts[2]
    kind = "vec"
    for k in ("skinny", "realign", "narrow", "ring", "dma"):
        if any(p.startswith(k) for p in parts[3:]):
            kind = k
            break
    return dtype, a == "ak", b == "bk", kind


def grid_for(load):
    """Tile rows and columns of a product with 256 * load tiles."""
    tm = 8 if load < 1 else 16 if load <= 2 else 32
    return tm, int(CUS * load) // tm


class Pool:
    """Device buffers per (dtype, role), grown on demand and filled with normal random values."""

    def __init__(self, torch):
        self.torch = torch
        self.bufs = {}

    def get(self, dtype, role, numel):
        t = self.torch
        key = (dtype, role)
        b = self.bufs.get(key)
        if b is None or b.numel() < numel:
            self.bufs.pop(key, None)
            t.cuda.empty_cache()
            tdt = {"bf16": t.bfloat16, "f16": t.float16, "f32": t.float32,
                   "e4m3": t.float8_e4m3fn}[dtype]
            g = t.Generator(device="cuda")
            g.manual_seed(1234 + len(self.bufs))
            b = t.randn(numel, device="cuda", generator=g, dtype=t.float32)
            if dtype != "e4m3":
                b = b.mul_(0.125)
            b = b.to(tdt)
            self.bufs[key] = b
        return b


def operand_strides(kmajor, rows, K, odd):
    """(stride along rows, stride along K) and the element count of one operand."""
    if kmajor:
        ld = K + (1 if odd else 0)
        return (ld, 1), rows * ld
    ld = rows + (1 if odd else 0)
    return (1, ld), K * ld


def time_launches(H, torch, g, A, B, D, ws, reps, warmup=2):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.run(A, B, None, D, stream=stream, workspace=ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.run(A, B, None, D, stream=stream, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps   # microseconds per launch


def run_case(H, torch, pool, idx, dtype, ak, bk, odd, M, N, K, reps, split_k=1, decomposition=1,
             ldd=None):
    out_t = "bf16" if dtype == "e4m3" else dtype
    ldd = N if ldd is None else ldd
    a_str, a_n = operand_strides(ak, M, K, odd)
    b_rows_str, b_n = operand_strides(bk, N, K, odd)
    # B is K x N: make_desc takes (stride_k, stride_n)
    b_str = (b_rows_str[1], b_rows_str[0])
    A = pool.get(dtype, "A", a_n)
    B = pool.get(dtype, "B", b_n)
    D = pool.get(out_t, "D", M * ldd)
    desc = H.make_desc(M, N, K, dtype, a_str, b_str, (ldd, 1), force_config=idx, split_k=split_k,
                       decomposition=decomposition)
    g = H.Gemm(desc)
    try:
        ws = None
        if g.workspace_bytes:
            ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda")
        info = g.info
        return time_launches(H, torch, g, A, B, D, ws, reps), info
    finally:
        g.close()


def fit(t1, t2):
    c = (t2 - t1) / (KT[1] - KT[0])
    f = t1 - c * KT[0]
    return max(f, 0.0), max(c, 1e-4)


def entry_tile(H, torch, pool, idx, name):
    """(bm, bn, bk) of an entry, from a handle on a small product it fits."""
    dtype, ak, bk, kind = parse_name(name)
    probe_k = 4096 if dtype == "e4m3" else 2048
    _, info = run_case(H, torch, pool, idx, dtype, ak, bk, kind in ("realign", "narrow"), 512, 512,
                       probe_k, 1)
    return info.bm, info.bn, info.bk


def time_entry(H, torch, pool, idx, name, tile, reps):
    """Launch times (microseconds) at every load and both depths: [[t(kt1), t(kt2)] per load]."""
    dtype, ak, bk, kind = parse_name(name)
    odd = kind in ("realign", "narrow")
    bm, bn, bkk = tile
    out = []
    for load in LOADS:
        tm, tn = grid_for(load)
        times = []
        for kt in KT:
            t, inf = run_case(H, torch, pool, idx, dtype, ak, bk, odd, tm * bm, tn * bn, kt * bkk,
                              reps)
            assert inf.config == idx or inf.fallback == idx, (name, inf.name)
            times.append(t)
        out.append(times)
    return out


EDGE_KT = 32   # depth of the edge measurements, in k-tiles


def time_edges(H, torch, pool, idx, name, tile, reps):
    """Launch times (microseconds) at load 1 and EDGE_KT k-tiles: aligned; with a partial last
    k-tile; with a partial last tile row (8 rows) and column (8 columns short); with D's rows
    off 16 bytes (leading dimension N + 1)."""
    dtype, ak, bk, kind = parse_name(name)
    odd = kind in ("realign", "narrow")
    bm, bn, bkk = tile
    M, N, K = 16 * bm, 16 * bn, EDGE_KT * bkk
    out = []
    for m, n, k, ldd in ((M, N, K, N), (M, N, K - bkk // 2, N), (M - bm + 8, N - 8, K, N - 8),
                         (M, N, K, N + 1)):
        t, inf = run_case(H, torch, pool, idx, dtype, ak, bk, odd, m, n, k, reps, ldd=ldd)
        assert inf.config == idx or inf.fallback == idx, (name, inf.name)
        out.append(t)
    return out


def calibrate_split(H, torch, pool, costs, names, reps):
    """Residual time of split-K runs (second kernel and partial stores) against the entry's own
    prediction, fitted to g0 + g1 * bytes by least squares."""
    import numpy as np
    cases = [("bf16_ak_bk_256x256x64_w2x4_m16_ring", 1536, 1536, 8192, (2, 4, 7)),
             ("bf16_ak_bk_256x256x64_w2x4_m16_ring", 2048, 2048, 4096, (2, 4)),
             ("bf16_ak_bk_128x128x64_w2x2_m32_vec", 512, 512, 16384, (4, 8, 16)),
             ("bf16_ak_bk_128x128x64_w2x2_m32_vec", 1024, 1024, 8192, (2, 4, 8)),
             ("f16_ak_bk_256x256x64_w2x4_m16_ring", 2816, 2816, 4096, (2,)),
             ("e4m3_ak_bk_256x256x128_w2x4_m32_ring", 1536, 1536, 16384, (2, 4, 7))]
    X, y = [], []
    for name, M, N, K, splits in cases:
        if name not in costs:
            continue
        idx = names.index(name)
        dtype, ak, bk, _ = parse_name(name)
        out_sz = 4 if dtype == "f32" else 2
        for s in splits:
            t, info = run_case(H, torch, pool, idx, dtype, ak, bk, False, M, N, K, reps, split_k=s)
            S = info.split_k
            kt = -(-K // (info.bk * S)) if S > 1 else -(-K // info.bk)
            wg = -(-M // info.bm) * -(-N // info.bn) * S
            pred = predict(costs[name], wg, kt)
            nbytes = 2 * S * M * N * 4 + M * N * out_sz
            X.append([1.0, nbytes])
            y.append(t - pred)
            print(f"split {name} {M}x{N}x{K} S={S}: {t:.1f} us, entry model {pred:.1f}", flush=True)
    (g0, g1), *_ = np.linalg.lstsq(np.array(X), np.array(y), rcond=None)
    return max(float(g0), 0.0), max(float(g1), 0.0)


def predict(rows, wg, kt):
    """The chooser's time (microseconds) for a launch of wg workgroups of kt k-tiles each, the
    same formula as the library's: whole loads n (n workgroups on every compute unit) take the
    measured time, a load above 8 adds whole groups of 8, and a partly filled last round costs
    the step to the next whole load, scaled as a round with that fraction of the units busy."""
    if wg <= 0 or kt <= 0:
        return 0.0

    def at(i):
        return rows[i][0] + kt * rows[i][1]

    def whole(n):
        if n <= 0:
            return 0.0
        g = (n - 1) // 8
        return g * at(len(LOADS) - 1) + at(n - 8 * g + ONE - 1)

    def part(w):
        # piecewise linear over the loads below one, relative to a full round
        if w <= LOADS[0]:
            t = at(0)
        else:
            i = 1
            while LOADS[i] < w:
                i += 1
            lo, hi = LOADS[i - 1], LOADS[i]
            t = at(i - 1) + (w - lo) / (hi - lo) * (at(i) - at(i - 1))
        return t / at(ONE)

    n = -(-wg // CUS)
    w = (wg - (n - 1) * CUS) / CUS
    lo, hi = whole(n - 1), whole(n)
    return lo + (hi - lo) * part(w)


def calibrate_sk(H, torch, pool, costs, names, reps):
    """Stream-K runs against the prediction for their whole tiles; the rest is fitted to
    s0 + s1 * (the entry's time for 256 workgroups of one share of k-tiles)."""
    import numpy as np
    X, y = [], []
    for name in ("bf16_ak_bk_256x256x64_w2x4_m16_ring", "f16_ak_bk_256x256x64_w2x4_m16_ring",
                 "bf16_ak_bn_256x256x64_w2x4_m16_ring"):
        if name not in costs:
            continue
        idx = names.index(name)
        dtype, ak, bk, _ = parse_name(name)
        for tm, tn, kt in ((17, 16, 128), (19, 16, 64), (18, 20, 128), (24, 16, 64),
                           (20, 30, 64), (17, 17, 128), (24, 24, 128), (28, 28, 128)):
            t, info = run_case(H, torch, pool, idx, dtype, ak, bk, False, tm * 256, tn * 256,
                               kt * info_bk(dtype), reps, decomposition=2)
            tiles = tm * tn
            sk = info.sk_tiles
            whole = predict(costs[name], tiles - sk, kt)
            share = predict(costs[name], CUS, -(-sk * kt // CUS))
            X.append([1.0, share])
            y.append(t - whole)
            print(f"stream-k {name} {tiles} tiles ({sk} shared) x {kt} k-tiles: {t:.1f} us, "
                  f"whole tiles {whole:.1f}, one share {share:.1f}", flush=True)
    if len(X) < 2:
        return 10.0, 2.0
    (s0, s1), *_ = np.linalg.lstsq(np.array(X), np.array(y), rcond=None)
    return max(float(s0), 0.0), max(float(s1), 0.0)


def info_bk(dtype):
    """k-tile depth of the ring entries: 128 bytes of K."""
    return 128 if dtype == "e4m3" else 64 if dtype in ("bf16", "f16") else 32


def calibrate_repack(H, torch, pool, costs, names, reps):
    """Residual time of runs on aligned copies against the prediction for the inner product,
    fitted to h0 + h1 * bytes."""
    import numpy as np
    # fp8 has no realigning loader, so its small products run on copies whatever the table says:
    # they pin the fixed cost, which the large products alone leave to extrapolation
    cases = [("f16", 4099, 3071, 2053, True, False), ("bf16", 6001, 5003, 3001, True, False),
             ("e4m3", 3001, 2999, 2049, True, True), ("bf16", 8191, 8191, 4097, True, True),
             ("f16", 5003, 3001, 6007, False, False), ("e4m3", 2051, 1533, 1027, True, False),
             ("e4m3", 1001, 1003, 999, True, False)]
    X, y = [], []
    for dtype, M, N, K, ak, bk in cases:
        t, info = run_case(H, torch, pool, -1, dtype, ak, bk, True, M, N, K, reps, split_k=0)
        inner = info.name.decode()
        if not info.repack or inner not in costs:
            print(f"repack {dtype} {M}x{N}x{K}: not run on copies ({inner})", flush=True)
            continue
        esz = 1 if dtype == "e4m3" else 2
        kp = -(-K // (16 // esz)) * (16 // esz)
        S = info.split_k
        kt = -(-kp // (info.bk * S))
        wg = -(-M // info.bm) * -(-N // info.bn) * S
        pred = predict(costs[inner], wg, kt)
        pred += edge_time(EDGES[inner], M, N, kp, info.bm, info.bn, info.bk,
                          d_rows_aligned=(N * 2) % 16 == 0)
        if S > 1:
            pred += SPLIT[0] + SPLIT[1] * (2 * S * M * N * 4 + M * N * 2)
        nbytes = 2 * (M + N) * kp * esz
        X.append([1.0, nbytes])
        y.append(t - pred)
        print(f"repack {dtype} {M}x{N}x{K} -> {inner} S={S}: {t:.1f} us, inner model {pred:.1f}",
              flush=True)
    if len(X) < 2:
        return 5.0, 1.0 / 3.6e6
    (h0, h1), *_ = np.linalg.lstsq(np.array(X), np.array(y), rcond=None)
    return max(float(h0), 0.0), max(float(h1), 0.0)


def edge_time(edges, M, N, K, bm, bn, bk, d_rows_aligned=True):
    """The library's edge terms: a partial last k-tile costs edges[0] per workgroup on the busiest
    compute unit, partial last tile rows or columns edges[1] once, D rows off 16 bytes edges[2]
    per workgroup on the busiest compute unit."""
    tiles = -(-M // bm) * -(-N // bn)
    per_cu = -(-tiles // CUS)
    t = edges[0] * per_cu if K % bk else 0.0
    t += edges[2] * per_cu if not d_rows_aligned else 0.0
    return t + (edges[1] if M % bm or N % bn else 0.0)


SPLIT = [0.0, 0.0]
EDGES = {}


def emit(costs, edges, split, repack, sk, device, out):
    lines = [
        "// cost_table.cpp -- measured cost model of the tile table (MI355X), written by",
        "// hierarchical_tiling_amd/calibrate.py; do not edit by hand.",
        f"// Device: {device}.",
        "// For each entry, index i = 0..10 stands for the load 1/4, 1/2, 3/4, 1, 2, ..., 8",
        "// (workgroups per compute unit): a launch of 256 * load workgroups of kt k-tiles each",
        "// takes f[i] + kt * c[i] microseconds.  Then the extra time of a partial last k-tile",
        "// (per workgroup on the busiest compute unit), of partial last tile rows and columns",
        "// (once), and of D rows off 16 bytes (per workgroup on the busiest compute unit).",
        '#include "gemm_internal.h"',
        "",
        "namespace htk {",
        "",
        "const EntryCost kEntryCosts[] = {",
    ]
    for name, rows in costs.items():
        fs = ", ".join(f"{f:.2f}f" for f, _ in rows)
        cs = ", ".join(f"{c:.4f}f" for _, c in rows)
        ek, emn, ed = edges[name]
        lines.append(f'    {{"{name}",\n     {{{fs}}},\n     {{{cs}}},\n     {ek:.2f}f, {emn:.2f}f, '
                     f'{ed:.2f}f}},')
    lines += [
        "};",
        "const int kEntryCostCount = (int)(sizeof(kEntryCosts) / sizeof(kEntryCosts[0]));",
        "",
        "// split-K second kernel and partial stores: g0 + g1 * bytes microseconds",
        f"const double kSplitFixedUs = {split[0]:.3f};",
        f"const double kSplitUsPerByte = {split[1]:.6e};",
        "// copies of A and B into aligned K-major buffers: h0 + h1 * bytes microseconds",
        f"const double kRepackFixedUs = {repack[0]:.3f};",
        f"const double kRepackUsPerByte = {repack[1]:.6e};",
        "// Stream-K launch and fix-up beyond the whole tiles: s0 + s1 * (the entry's time for 256",
        "// workgroups of one share of k-tiles) microseconds",
        f"const double kSkFixedUs = {sk[0]:.3f};",
        f"const double kSkShareFactor = {sk[1]:.4f};",
        "",
        "}  // namespace htk",
        "",
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))


def check_shapes():
    """(dtype, M, N, K, A K-major, B K-major, odd leading dimensions) of the choice check: the
    benchmark's products, square and skinny ones, odd leading dimensions, and seeded random ones."""
    import random
    S = [("bf16", 8192, 8192, 8192, True, True, False), ("bf16", 8192, 8192, 8192, True, False, False),
         ("bf16", 4096, 4096, 4096, True, True, False), ("e4m3", 8192, 8192, 8192, True, True, False),
         ("f16", 4099, 3071, 2053, True, False, True), ("f32", 256, 256, 256, True, False, False)]
    for M, N, K in [(3072, 3072, 3072), (2816, 2816, 4096), (1536, 1536, 8192), (2048, 2048, 4096),
                    (2048, 4096, 2048), (512, 512, 16384), (4352, 4352, 4096), (6144, 6144, 8192),
                    (1024, 1024, 1024), (768, 768, 4096), (256, 4096, 4096)]:
        S.append(("bf16", M, N, K, True, True, False))
    for M, N, K in [(1001, 999, 1003), (2051, 1533, 1027), (1503, 1301, 1101)]:
        S.append(("f16", M, N, K, True, False, True))
    S += [("e4m3", 3001, 2999, 2049, True, True, True), ("e4m3", 2048, 2048, 8192, True, True, False),
          ("f32", 1536, 1536, 1536, True, False, False)]
    rng = random.Random(7)
    for _ in range(16):
        dt = rng.choice(["bf16", "bf16", "f16", "e4m3"])
        M = rng.randrange(200, 6000) // 8 * 8
        N = rng.randrange(200, 6000) // 8 * 8
        K = rng.randrange(256, 8192) // 64 * 64
        S.append((dt, M, N, K, True, dt == "e4m3" or rng.random() < 0.6, False))
    return S


def check(H, torch, pool, names, reps, out):
    """Times the automatic choice and every fitting entry (each with the plan the library gives
    it) on check_shapes(); prints the automatic choice's time over the best measured one and
    their geometric mean."""
    import math
    lines, logsum, n = [], 0.0, 0
    for dt, M, N, K, ak, bk, odd in check_shapes():
        t_auto, info = run_case(H, torch, pool, -1, dt, ak, bk, odd, M, N, K, reps, split_k=0,
                                decomposition=0)
        best, best_name = t_auto, info.name.decode()
        for i, name in enumerate(names):
            d_, ak_, bk_, kind = parse_name(name)
            if d_ != dt or ak_ != ak or bk_ != bk or kind == "skinny":
                continue
            try:
                t, _ = run_case(H, torch, pool, i, dt, ak, bk, odd, M, N, K, reps, split_k=0,
                                decomposition=0)
            except H.GemmError:
                continue       # the entry does not fit this product
            if t < best:
                best, best_name = t, name
        logsum += math.log(t_auto / best)
        n += 1
        line = (f"{dt} {M}x{N}x{K} {'ak' if ak else 'am'}_{'bk' if bk else 'bn'}"
                f"{' odd' if odd else ''}: auto {info.name.decode()} S{info.split_k}"
                f"{' copies' if info.repack else ''} {t_auto:.1f} us (predicted "
                f"{info.predicted_us:.1f}); best {best_name} {best:.1f} us; ratio {t_auto / best:.3f}")
        print(line, flush=True)
        lines.append(line)
    summary = f"{n} products: geometric mean of automatic / best = {math.exp(logsum / n):.4f}"
    print(summary, flush=True)
    with open(out, "w") as fh:
        fh.write("\n".join(lines + [summary]) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--check", action="store_true",
                    help="instead of measuring the table, time the automatic choice against every "
                         "fitting entry on a set of products and write the comparison to --out")
    ap.add_argument("--only", default=None, help="regular expression over entry names")
    ap.add_argument("--reps", type=int, default=16)
    ap.add_argument("--passes", type=int, default=5)
    args = ap.parse_args(argv)
    import torch

    from hierarchical_tiling_amd import htgemm as H
    if not torch.cuda.is_available():
        sys.exit("calibration needs the GPU")
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    pool = Pool(torch)
    if args.check:
        check(H, torch, pool, names, args.reps, args.out)
        return
    import numpy as np
    chosen = [(i, n) for i, n in enumerate(names) if parse_name(n)[3] != "skinny" and
              (not args.only or re.search(args.only, n))]
    tiles = {n: entry_tile(H, torch, pool, i, n) for i, n in chosen}
    raw = {n: [] for _, n in chosen}
    raw_edges = {n: [] for _, n in chosen}
    t0 = time.time()
    # whole passes over the table, so that drifts of clock and temperature fall on every entry
    for p in range(args.passes):
        for idx, name in chosen:
            raw[name].append(time_entry(H, torch, pool, idx, name, tiles[name], args.reps))
            raw_edges[name].append(time_edges(H, torch, pool, idx, name, tiles[name], args.reps))
        print(f"[{time.time() - t0:6.1f} s] pass {p + 1} of {args.passes}", flush=True)
    costs, edges = {}, {}
    for _, name in chosen:
        med = np.median(np.array(raw[name]), axis=0)    # loads x depths
        costs[name] = [fit(t1, t2) for t1, t2 in med]
        ta, tk, tmn, td = np.median(np.array(raw_edges[name]), axis=0)
        edges[name] = tuple(max(float(t - ta), 0.0) for t in (tk, tmn, td))
        print(f"{name}: " + " ".join(f"{f:.1f}+{c:.3f}k" for f, c in costs[name]) +
              "  edges k %.1f mn %.1f d %.1f" % edges[name], flush=True)
    EDGES.update(edges)
    split = calibrate_split(H, torch, pool, costs, names, args.reps)
    SPLIT[:] = split
    print(f"split: {split[0]:.2f} us + {split[1]:.3e} us/B", flush=True)
    repack = calibrate_repack(H, torch, pool, costs, names, args.reps)
    print(f"repack: {repack[0]:.2f} us + {repack[1]:.3e} us/B", flush=True)
    sk = calibrate_sk(H, torch, pool, costs, names, args.reps)
    print(f"stream-k: {sk[0]:.2f} us + {sk[1]:.3f} x share", flush=True)
    props = torch.cuda.get_device_properties(0)
    device = f"{props.gcnArchName.split(':')[0]}, {props.multi_processor_count} compute units"
    emit(costs, edges, split, repack, sk, device, args.out)
    print(f"wrote {args.out}", flush=True)


if __name__ == "__main__":
    main()
