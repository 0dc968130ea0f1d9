"""Benchmark of the hierarchically tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-sub]
                    [--no-cpu-baseline]

A step is one launch of the whole hot path -- D = act(alpha*(A@B) + beta*C + bias) -- over one
set of synthetic inputs already resident in HBM.  The default workload is the headline one:
bf16 8192 x 8192 x 8192, A row-major, B column-major, D = GELU(A@B + bias[n]), fp32 accumulate,
bf16 output; `value` is its throughput.  The other benchmark workloads are timed after it the same
way and reported as `sub_results`, each with its own roofline fraction.  Input sets are rotated
so that consecutive steps do not find their operands in the 256 MiB last-level cache.  Prints one
JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
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
    "bf16_8192_gelu_bn": (8192, 8192, 8192, "bf16", "row", "row", "normal", 8192 ** -0.5, 1.0,
                          0.0, False, True, "gelu", 1.0, 1.0),
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
    "bf16_8192_gelu_bn": "bf16 GEMM 8192x8192x8192, D=GELU(A@B+bias[n]), A row-major, B row-major, fp32 accumulate, bf16 out",
    "bf16_4096": "bf16 GEMM 4096x4096x4096, D=A@B, A row-major, B column-major, bf16 out",
    "fp16_ragged": "fp16 GEMM 4099x3071x2053, D=0.75*A@B-1.25*C, A/B/C row-major (odd leading dims)",
    "e4m3_skinny": "e4m3 GEMM 16x16384x8192, D=sA*sB*A@B, A row-major, B column-major, bf16 out",
    "e4m3_8192": "e4m3 GEMM 8192x8192x8192, D=sA*sB*A@B, A row-major, B column-major, bf16 out",
    "fp32_256": "fp32 GEMM 256x256x256, D=1.5*A@B+0.5*C, all row-major",
}
SEEDS = {"bf16_8192_gelu": 4000, "bf16_8192_gelu_bn": 4200, "bf16_4096": 2000,
         "fp16_ragged": 3000, "e4m3_skinny": 5000, "e4m3_8192": 5100, "fp32_256": 1000}
# input sets rotated per workload: at least 512 MiB of operands (twice the last-level cache)
# wherever the operands are that large
SETS = {"bf16_8192_gelu": 3, "bf16_8192_gelu_bn": 3, "bf16_4096": 6, "fp16_ragged": 6,
        "e4m3_skinny": 4, "e4m3_8192": 4, "fp32_256": 1}
# the HBM-bound workload (its roofline is bytes, not FLOPs)
MEMORY_BOUND = {"e4m3_skinny"}
SUB_WORKLOADS = ["e4m3_skinny", "e4m3_8192", "bf16_4096", "fp16_ragged", "bf16_8192_gelu_bn",
                 "fp32_256"]


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
        host.append((A, B, C, bv) if s == 0 else None)   # the host copy of set 0 feeds the oracle
        sets.append(tuple(inputs.to_device(x, device) if x is not None else None for x in (A, B, C, bv)))
    D = torch.empty(M * N * inputs.ESIZE[out_t], dtype=torch.uint8, device=device)
    return host, sets, D


def measure(name, steps, warmup, device, clock_sampler=None):
    """Time `steps` back-to-back launches of workload `name` after `warmup` untimed ones."""
    import torch

    from hierarchical_tiling_amd import counters
    from hierarchical_tiling_amd import htgemm as H
    M, N, K, dt, ao, bo, dist, std, alpha, beta, has_c, bias, act, sa, sb = WORKLOADS[name]
    host, sets, D = build_inputs(name, SETS[name], device)
    A0, B0, C0, _ = host[0]
    desc = H.make_desc(M, N, K, dt, A0.strides, B0.strides, (N, 1),
                       c_strides=C0.strides if C0 is not None else None, has_bias=bias, act=act)
    g = H.Gemm(desc)
    info = g.info
    ws = None
    if g.workspace_bytes:
        ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()

    def step(i):
        a, b, c, bv = sets[i % len(sets)]
        g.run(a, b, c, D, bv, alpha=alpha, beta=beta, scale_a=sa, scale_b=sb, stream=stream,
              workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: the launches back to back on the launch stream, one pair of HIP events
    # around them (events between launches would add their own gaps to short kernels)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    launch_ms = float(t_start.elapsed_time(t_end)) / steps
    # spread of single launches, in a separate pass (not part of the value)
    n_pct = min(steps, 20)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_pct)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_pct)]
    for i in range(n_pct):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    kclock = kernel_clock(H, g, info, step) if clock_sampler is not None else None
    clock = None
    if clock_sampler is not None and not isinstance(clock_sampler, NoSampler):
        # shader clock while the kernel runs back to back for about a second (its own pass)
        n_sus = max(1, int(1000.0 / max(launch_ms, 1e-3)))
        with clock_sampler:
            for i in range(n_sus):
                step(i)
            torch.cuda.synchronize()
        clock = clock_sampler.summary()
    flops = 2.0 * M * N * K
    nbytes = algorithmic_bytes(M, N, K, dt, has_c, bias)
    if name in MEMORY_BOUND:
        ach = nbytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = flops / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[dt],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[dt], 4)}
    kname = info.name.decode()
    traffic, source = counters.traffic_for(kname, name, os.path.join(ROOT, "profiles"))
    roof["traffic"] = traffic
    roof.update({"traffic_source": source, "kernel": kname, "launch_ms_mean": round(launch_ms, 4),
                 "single_launch_ms_p10": round(float(np.percentile(per, 10)), 4),
                 "single_launch_ms_p50": round(float(np.percentile(per, 50)), 4),
                 "single_launch_ms_p90": round(float(np.percentile(per, 90)), 4),
                 "algorithmic_bytes": nbytes, "algorithmic_flops": flops})
    res = {"workload": DESCRIBE[name], "name": name, "M": M, "N": N, "K": K, "dtype": dt,
           "tile": [info.bm, info.bn, info.bk], "grid": int(info.grid), "split_k": int(info.split_k),
           "steps": steps, "warmup": warmup, "input_sets": SETS[name], "ms_per_step": round(wall_ms, 4),
           "tflops": round(flops / (wall_ms * 1e-3) / 1e12, 1), "roofline": roof}
    if clock is not None:
        res["sclk_mhz_during_sustained_run"] = clock
    if kclock is not None:
        mhz = kclock["median"]
        peak_at = roof["peak"] * mhz / MAX_SCLK_MHZ
        kclock["peak_at_this_clock"] = round(peak_at, 1)
        kclock["frac_at_this_clock"] = round(roof["achieved"] / peak_at, 4)
        res["sclk_mhz_in_kernel"] = kclock
    return res, host[0]


def kernel_clock(H, g, info, step, launches=10):
    """The shader clock the product kernel ran at, from its own counters: the handle's clock
    record (gemm_set_clock_record) over `launches` back-to-back launches after the timed region;
    the last launch's per-workgroup records give (shader cycles) / (real-time ticks) x 100 MHz.
    None where the chosen kernel does not record."""
    import torch
    if not info.name.decode().endswith("_pp"):
        return None
    n = int(info.grid)
    rec = torch.zeros(4 * n, dtype=torch.int64, device="cuda")
    H.gemm_set_clock_record(g.handle, rec, n)
    for i in range(launches):
        step(i)
    torch.cuda.synchronize()
    H.gemm_set_clock_record(g.handle, None, 0)
    r = rec.cpu().numpy().astype(np.float64).reshape(n, 4)
    ok = (r[:, 3] > r[:, 2]) & (r[:, 1] > r[:, 0])
    if not ok.any():
        return None
    mhz = (r[ok, 1] - r[ok, 0]) / (r[ok, 3] - r[ok, 2]) * REALTIME_MHZ
    return {"median": round(float(np.median(mhz)), 1), "p10": round(float(np.percentile(mhz, 10)), 1),
            "p90": round(float(np.percentile(mhz, 90)), 1), "workgroups": int(ok.sum()),
            "launches": launches, "method": "s_memtime / s_memrealtime per workgroup, last launch"}


# the constant-rate counter that s_memrealtime reads, and the maximum shader clock (MI355X)
REALTIME_MHZ = 100.0
MAX_SCLK_MHZ = 2400.0


class NoSampler:
    """Stands in for ClockSampler where only the in-kernel clock is wanted."""

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False

    def summary(self):
        return None


class ClockSampler:
    """Samples the GPU's current graphics clock (amdsmi, in-process) every few milliseconds while
    it is entered; summary() gives the median and range in MHz, or None if unavailable."""

    def __init__(self):
        self.samples = []
        self._stop = threading.Event()
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._amdsmi = amdsmi
            self._handle = handles[0] if handles else None
        except Exception:
            self._handle = None

    def _read(self):
        info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
        return float(info.get("clk", info.get("cur_clk")))

    def __enter__(self):
        self.samples = []
        self._stop.clear()
        if self._handle is not None:
            def run():
                while not self._stop.is_set():
                    try:
                        self.samples.append(self._read())
                    except Exception:
                        return
                    time.sleep(0.005)
            self._t = threading.Thread(target=run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._handle is not None:
            self._t.join(timeout=2)
        return False

    def max_mhz(self):
        try:
            info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
            return float(info.get("max_clk"))
        except Exception:
            return None

    def summary(self):
        if not self.samples:
            return None
        s = np.array(self.samples)
        return {"median": float(np.median(s)), "min": float(s.min()), "max": float(s.max()),
                "samples": int(s.size), "max_sclk": self.max_mhz()}


def run_metadata(threads):
    import torch
    props = torch.cuda.get_device_properties(0)
    meta = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hbm_gib": round(props.total_memory / 2 ** 30, 1),
            "torch": torch.__version__, "torch_hip": torch.version.hip}
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    # the compiler that built the library (recorded by the build; no child process here, which
    # under a profiler's preload would start a second GPU client)
    try:
        with open(os.path.join(ROOT, "hierarchical_tiling_amd", "libhtgemm.so.buildinfo")) as f:
            meta.update(json.loads(f.read()))
    except Exception:
        meta["hipcc"] = None
    try:
        import ctypes
        v = ctypes.c_int()
        ctypes.CDLL("libamdhip64.so").hipRuntimeGetVersion(ctypes.byref(v))
        meta["hip_runtime_version"] = v.value
    except Exception:
        meta["hip_runtime_version"] = None
    try:
        meta["cpu_model"] = next(line.split(":", 1)[1].strip() for line in open("/proc/cpuinfo")
                                 if line.startswith("model name"))
    except Exception:
        meta["cpu_model"] = None
    meta["host_cpus_available"] = len(os.sched_getaffinity(0))
    meta["host_threads_used"] = threads
    return meta


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
    ap.add_argument("--no-sub", action="store_true", help="time only --workload")
    ap.add_argument("--sub-steps", type=int, default=30)
    ap.add_argument("--sub-warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the one-second sustained run that samples the shader clock")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain device copies of 1 GiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    dev = torch.device("cuda:0")
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    sampler = None if args.no_clock else ClockSampler()
    main_res, host0 = measure(args.workload, args.steps, args.warmup, dev, clock_sampler=sampler)
    torch.cuda.empty_cache()
    subs = []
    if not args.no_sub:
        for name in SUB_WORKLOADS:
            if name == args.workload:
                continue
            r, _ = measure(name, args.sub_steps, args.sub_warmup, dev,
                           clock_sampler=NoSampler() if not args.no_clock else None)
            subs.append(r)
            torch.cuda.empty_cache()
    name = args.workload
    M, N, K, dt = WORKLOADS[name][:4]
    out = {
        "metric": METRIC, "value": main_res["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded numpy PCG64 draws rounded to the operand type)",
        "config": {"workload": DESCRIBE[name], "M": M, "N": N, "K": K, "tile": main_res["tile"],
                   "grid": main_res["grid"], "input_sets": SETS[name]},
        "roofline": main_res["roofline"],
        "sclk_mhz_during_sustained_run": main_res.get("sclk_mhz_during_sustained_run"),
        "sclk_mhz_in_kernel": main_res.get("sclk_mhz_in_kernel"),
        "sub_results": subs,
        "run": run_metadata(threads),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, host0, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
