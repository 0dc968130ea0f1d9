"""Build libhtgemm.so (gfx950 HIP kernels + host API + layout helper) in the package directory.

    python -m hierarchical_tiling_amd.build [--incremental]

Objects go to _build/ at the repository root; the shared library lands next to this file so the
binding loads it in-tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhtgemm.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions are kept out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument"]

HIP = [HIPCC, f"--offload-arch={ARCH}"] + COMMON + DEVICE_FLAGS
# kernels.h holds the kernel templates; each table_*.hip instantiates one operand type's entries
SOURCES = [
    ("table_bf16.hip", HIP),
    ("table_bf16_dma.hip", HIP),
    ("table_f16.hip", HIP),
    ("table_e4m3.hip", HIP),
    ("table_f32.hip", HIP),
    ("table_pp.hip", HIP),
    ("table.cpp", HIP),
    ("cost_table.cpp", HIP),
    ("reduce.hip", HIP),
    ("probe.hip", HIP),
    ("repack.hip", HIP),
    ("api.cpp", HIP),
    ("layout.cpp", ["g++"] + COMMON),
]


HEADERS = [os.path.join(CSRC, "kernels.h"), os.path.join(CSRC, "pingpong.h"), os.path.join(CSRC, "gemm_internal.h"),
           os.path.join(CSRC, "atom_maps.h"),
           os.path.join(ROOT, "include", "htgemm.h"), os.path.join(ROOT, "include", "htlayout.h")]


def _compile(src, cmd, incremental=False):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(f) for f in HEADERS + [os.path.join(CSRC, src)])
        if os.path.getmtime(obj) > newest:
            return obj
    full = cmd + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(full, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(full)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (incremental=True skips objects newer than their source and the
    shared headers) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda sc: _compile(sc[0], sc[1], incremental), SOURCES))
    tmp = OUT + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    # the compiler that built the library, for the benchmark's run record
    ver = subprocess.run([HIPCC, "--version"], capture_output=True, text=True).stdout.splitlines()
    with open(OUT + ".buildinfo", "w") as f:
        f.write(json.dumps({"hipcc": next((v for v in ver if v.startswith("HIP version")), None),
                            "clang": next((v for v in ver if "clang version" in v), None),
                            "offload_arch": ARCH}) + "\n")
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
    sys.exit(0)
