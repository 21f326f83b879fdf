"""Build libw8a8.so (HIP for gfx950) in-tree with hipcc.

    python w8a8_int8_dynamic_amd/build.py [--jobs N] [--save-temps]

(run as a script, or through __graft_entry__.build(): importing the package
loads the library, which may not exist yet)

Each source is compiled to an object under ``_build/`` in parallel, then
linked into ``w8a8_int8_dynamic_amd/libw8a8.so``. Floating-point flags are
fixed: no fast-math, no contraction (the epilogue's rounding order is part
of the result), and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libw8a8.so")
SOURCES = ["quant.hip", "prepack.hip", "scaled_mm.hip", "scaled_mm_fp8.hip", "skinny_mm.hip", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libw8a8")
    return path


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, save_temps: bool = False, verbose: bool = False) -> str:
    """Compile every source and link libw8a8.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-save-temps"] if save_temps else []
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libw8a8.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--jobs", type=int, default=min(4, os.cpu_count() or 1))
    p.add_argument("--save-temps", action="store_true")
    args = p.parse_args(argv)
    build(args.jobs, args.save_temps, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
