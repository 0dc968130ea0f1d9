"""HBM bytes per launch from rocprofv3 counter collections.

Two `rocprofv3 --pmc` runs of the same command, one collecting FETCH_SIZE and one WRITE_SIZE
(KiB per dispatch, summed over the L2 channels), give the bytes a kernel moved between L2 and
memory.  Each counter is scaled by the factor that makes it read right for a plain device copy of
known size (bytes actually copied / counter reading), taken from two more runs of
`bench.py --copy-calibration`.  The result is written as a short text summary under `profiles/`
together with the kernel's name and a digest of the kernel source it was measured on; bench.py
reports the figure only while that digest still matches, so a changed kernel reports null.

    python -m hierarchical_tiling_amd.counters --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --kernel NAME --workload W --command "..." \
        --out profiles/<kernel>_<workload>_traffic.txt
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ("csrc/kernels.h", "csrc/pingpong.h", "csrc/gemm_internal.h", "csrc/atom_maps.h")
COPY_BYTES_DEFAULT = 1 << 30


def source_digest() -> str:
    """sha256 over the kernel sources (a change to any kernel invalidates stored counters)."""
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def per_dispatch(path: str, counter: str) -> dict[str, list[float]]:
    """kernel name -> counter value of each of its dispatches (in dispatch order)."""
    vals: dict[tuple[str, int], float] = defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[(r["Kernel_Name"], int(r["Dispatch_Id"]))] += float(r["Counter_Value"])
    out: dict[str, list[float]] = defaultdict(list)
    for (name, _), v in sorted(vals.items(), key=lambda kv: kv[0][1]):
        out[name].append(v)
    return out


def kernel_values(path: str, counter: str, kernel: str) -> list[float]:
    """Values of the dispatches whose demangled name contains `kernel`."""
    got = [v for name, vs in per_dispatch(path, counter).items() if kernel in name for v in vs]
    if not got:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} with {counter} in {path}")
    return got


def copy_factor(path: str, counter: str, copy_bytes: int, copies: int) -> float:
    """Bytes per counter byte for the calibration copies (all copyBuffer dispatches together)."""
    vals = kernel_values(path, counter, "copyBuffer")
    kib = sum(vals)
    return copy_bytes * copies / (kib * 1024.0)


def summarize(a) -> dict:
    fetch = kernel_values(a.fetch, "FETCH_SIZE", a.kernel_match)
    write = kernel_values(a.write, "WRITE_SIZE", a.kernel_match)
    ff = copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_bytes, a.copies)
    fw = copy_factor(a.copy_write, "WRITE_SIZE", a.copy_bytes, a.copies)
    fetch_kib = sum(fetch) / len(fetch)
    write_kib = sum(write) / len(write)
    return {
        "kernel": a.kernel, "workload": a.workload, "source_digest": source_digest(),
        "dispatches": [len(fetch), len(write)],
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
        "copy_bytes": a.copy_bytes, "copies": a.copies,
        "fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
        "traffic_bytes": int(fetch_kib * 1024 * ff + write_kib * 1024 * fw),
        "command": a.command,
    }


def write_summary(path: str, s: dict) -> None:
    lines = [
        f"# HBM traffic of {s['kernel']} on {s['workload']}",
        "",
        "rocprofv3 --pmc, one counter per run; values are KiB per dispatch, mean over dispatches.",
        "Each counter is scaled by bytes/counter of a plain device copy of known size.",
        "",
        f"command: {s['command']}",
        "",
        "```json",
        json.dumps(s, indent=1),
        "```",
        "",
    ]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def load(path: str) -> dict | None:
    """The JSON block of a summary written by write_summary, or None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    try:
        body = text.split("```json", 1)[1].split("```", 1)[0]
        return json.loads(body)
    except (IndexError, ValueError):
        return None


def traffic_for(kernel: str, workload: str, profiles_dir: str) -> tuple[int | None, str | None]:
    """(bytes per launch, summary file) when a summary for this kernel and workload exists and
    was measured on the current kernel sources; (None, reason) otherwise."""
    path = os.path.join(profiles_dir, f"{kernel}_{workload}_traffic.txt")
    s = load(path)
    if s is None:
        return None, "no counter summary"
    if s.get("kernel") != kernel or s.get("source_digest") != source_digest():
        return None, "kernel changed since the counters were taken"
    return int(s["traffic_bytes"]), os.path.relpath(path, os.path.dirname(profiles_dir))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--kernel", required=True, help="table entry name")
    ap.add_argument("--kernel-match", required=True, help="substring of the demangled kernel name")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--copy-bytes", type=int, default=COPY_BYTES_DEFAULT)
    ap.add_argument("--copies", type=int, default=5)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    s = summarize(a)
    write_summary(a.out, s)
    print(json.dumps(s))


if __name__ == "__main__":
    main()
