"""Build libmiattn.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_06_amd.build            # release library
    python -m exact_io_aware_06_amd.build --jobs 4

Each source compiles to an object in parallel, then one shared library is
linked next to this file, where the binding looks for it.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmiattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["miattn.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd.hip", "calib.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]
# Device code: keep the compiler from forming packed-fp32 VALU instructions.
HIP_FLAGS = ["-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libmiattn)")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS]
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    build(args.jobs)


if __name__ == "__main__":
    main()
