"""Benchmark of the hierarchically tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one launch of the whole hot path -- D = act(alpha*(A@B) + beta*C + bias) -- over one
set of synthetic inputs already resident in HBM.  The default workload is the headline one:
bf16 8192 x 8192 x 8192, A row-major, B column-major, D = GELU(A@B + bias[n]), fp32 accumulate,
bf16 output.  Three input sets are rotated so consecutive steps do not reuse the 256 MiB
last-level cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of gfx950 MFMA peak, bf16 8192³ D=αAB+βC"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    # name: (M, N, K, dtype, a_order, b_order, dist, std, alpha, beta, has_c, bias, act, sA, sB)
    "bf16_8192_gelu": (8192, 8192, 8192, "bf16", "row", "col", "normal", 8192 ** -0.5, 1.0, 0.0,
                       False, True, "gelu", 1.0, 1.0),
    "bf16_4096": (4096, 4096, 4096, "bf16", "row", "col", "normal", 4096 ** -0.5, 1.0, 0.0,
                  False, False, "none", 1.0, 1.0),
    "fp16_ragged": (4099, 3071, 2053, "f16", "row", "row", "uniform", None, 0.75, -1.25, True,
                    False, "none", 1.0, 1.0),
    "e4m3_skinny": (16, 16384, 8192, "e4m3", "row", "col", "normal", 1.0, 1.0, 0.0, False, False,
                    "none", 0.05, 0.05),
    "e4m3_8192": (8192, 8192, 8192, "e4m3", "row", "col", "normal", 1.0, 1.0, 0.0, False, False,
                  "none", 0.05, 0.05),
    "fp32_256": (256, 256, 256, "f32", "row", "row", "uniform", None, 1.5, 0.5, True, False,
                 "none", 1.0, 1.0),
}
DESCRIBE = {
    "bf16_8192_gelu": "bf16 GEMM 8192x8192x8192, D=GELU(A@B+bias[n]), A row-major, B column-major, fp32 accumulate, bf16 out",
    "bf16_4096": "bf16 GEMM 4096x4096x4096, D=A@B, A row-major, B column-major, bf16 out",
    "fp16_ragged": "fp16 GEMM 4099x3071x2053, D=0.75*A@B-1.25*C, A/B/C row-major (odd leading dims)",
    "e4m3_skinny": "e4m3 GEMM 16x16384x8192, D=sA*sB*A@B, A row-major, B column-major, bf16 out",
    "e4m3_8192": "e4m3 GEMM 8192x8192x8192, D=sA*sB*A@B, A row-major, B column-major, bf16 out",
    "fp32_256": "fp32 GEMM 256x256x256, D=1.5*A@B+0.5*C, all row-major",
}
SEEDS = {"bf16_8192_gelu": 4000, "bf16_4096": 2000, "fp16_ragged": 3000, "e4m3_skinny": 5000,
         "e4m3_8192": 5100, "fp32_256": 1000}


def algorithmic_bytes(M, N, K, dtype, has_c, bias):
    from hierarchical_tiling_amd.inputs import ESIZE
    out_t = "bf16" if dtype == "e4m3" else dtype
    e_in, e_out = ESIZE[dtype], ESIZE[out_t]
    return e_in * (M * K + K * N) + e_out * M * N * (2 if has_c else 1) + (e_out * N if bias else 0)


def build_inputs(name, n_sets, device):
    import torch

    from hierarchical_tiling_amd import inputs
    M, N, K, dt, ao, bo, dist, std, alpha, beta, has_c, bias, act, sa, sb = WORKLOADS[name]
    kw = {"std": std} if dist == "normal" else {}
    seed = SEEDS[name]
    host = []
    sets = []
    out_t = "bf16" if dt == "e4m3" else dt
    for s in range(n_sets):
        A = inputs.matrix(seed + 1 + 10 * s, M, K, dt, dist, order=ao, **kw)
        B = inputs.matrix(seed + 2 + 10 * s, K, N, dt, dist, order=bo, **kw)
        C = inputs.matrix(seed + 3 + 10 * s, M, N, out_t, "uniform", order="row") if has_c else None
        bv = inputs.vector(seed + 4 + 10 * s, N, out_t, "normal", std=0.1) if bias else None
        host.append((A, B, C, bv))
        sets.append(tuple(inputs.to_device(x, device) if x is not None else None for x in (A, B, C, bv)))
    D = torch.empty(M * N * inputs.ESIZE[out_t], dtype=torch.uint8, device=device)
    return host, sets, D


def cpu_baseline(name, host_set, threads, budget_s=12.0):
    """The oracle as it stands, timed on the host on a bounded sample of the same workload: the
    first m rows of D (all N columns, full K), m calibrated so the timed run lasts ~budget_s."""
    import oracle
    M, N, K, dt, ao, bo, dist, std, alpha, beta, has_c, bias, act, sa, sb = WORKLOADS[name]
    A, B, C, bv = host_set
    op = lambda m: oracle.Operand(m.storage, m.dtype, m.shape, m.strides) if m is not None else None  # noqa
    def rows_of(m):
        return np.repeat(np.arange(m), N), np.tile(np.arange(N), m)

    def run(m):
        r, c = rows_of(m)
        t0 = time.perf_counter()
        oracle.gemm_elems(op(A), op(B), r, c, op(C), op(bv), alpha=alpha, beta=beta, scale_a=sa,
                          scale_b=sb, act=act, threads=threads)
        return time.perf_counter() - t0

    m = 1
    t = run(m)
    while t < 0.5 and m < M:
        m = min(M, m * 4)
        t = run(m)
    m_final = int(min(M, max(1, m * budget_s / max(t, 1e-9))))
    t = run(m_final)
    flops = 2.0 * m_final * N * K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{m_final - 1} of D ({m_final}x{N} outputs, full K={K}), "
                      f"{t:.1f} s on {threads} threads",
            "seconds": round(t, 3)}


def copy_calibration(nbytes=1 << 30, copies=5):
    """Exactly `copies` device-to-device copies of `nbytes` and nothing else on the GPU: the
    reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"copy_bytes": nbytes, "copies": copies,
                      "GB/s (read+write)": round(2 * nbytes * copies / dt / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)  # untimed; lets the clock settle
    ap.add_argument("--workload", default="bf16_8192_gelu", choices=sorted(WORKLOADS))
    ap.add_argument("--force-config", type=int, default=-1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain device copies of 1 GiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from hierarchical_tiling_amd import htgemm as H
    dev = torch.device("cuda:0")
    name = args.workload
    M, N, K, dt, ao, bo, dist, std, alpha, beta, has_c, bias, act, sa, sb = WORKLOADS[name]
    host, sets, D = build_inputs(name, args.sets, dev)
    A0, B0, C0, _ = host[0]
    desc = H.make_desc(M, N, K, dt, A0.strides, B0.strides, (N, 1),
                       c_strides=C0.strides if C0 is not None else None, has_bias=bias, act=act,
                       force_config=args.force_config)
    g = H.Gemm(desc)
    info = g.info
    stream = torch.cuda.current_stream()

    def step(i):
        a, b, c, bv = sets[i % len(sets)]
        g.run(a, b, c, D, bv, alpha=alpha, beta=beta, scale_a=sa, scale_b=sb, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K launches back to back on the launch stream, one pair of HIP events around
    # them (per-launch events would add their own gaps to short kernels)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(wall * 1e3 / args.steps)
    avg_launch_ms = float(t_start.elapsed_time(t_end)) / args.steps
    # spread of single launches, in a separate pass (not part of the value)
    n_pct = min(args.steps, 20)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_pct)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_pct)]
    for i in range(n_pct):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms per launch
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    nbytes = algorithmic_bytes(M, N, K, dt, has_c, bias)
    memory_bound = name == "e4m3_skinny"
    if memory_bound:
        ach = nbytes / (avg_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS[dt],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[dt], 4), "traffic": None}
    from hierarchical_tiling_amd import counters
    traffic, source = counters.traffic_for(info.name.decode(), name, os.path.join(ROOT, "profiles"))
    roof["traffic"] = traffic
    roof.update({"traffic_source": source, "kernel": info.name.decode(),
                 "launch_ms_mean": round(avg_launch_ms, 4),
                 "single_launch_ms_p10": round(float(np.percentile(per, 10)), 4),
                 "single_launch_ms_p50": round(float(np.percentile(per, 50)), 4),
                 "single_launch_ms_p90": round(float(np.percentile(per, 90)), 4),
                 "algorithmic_bytes": nbytes, "algorithmic_flops": flops})
    out = {
        "metric": METRIC, "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded numpy PCG64 draws rounded to the operand type)",
        "config": {"workload": DESCRIBE[name], "M": M, "N": N, "K": K, "tile": [info.bm, info.bn, info.bk],
                   "grid": int(info.grid)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or min(16, len(os.sched_getaffinity(0)))
        out["cpu_baseline"] = cpu_baseline(name, host[0], threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
