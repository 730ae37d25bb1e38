"""Build libmiattn.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_06_amd.build            # release + race-detector libraries
    python -m exact_io_aware_06_amd.build --jobs 4 --sanitized

Each source compiles to an object in parallel, then the shared library is
linked next to this file, where the binding looks for it, together with
libmiattn_serial.so (the kernels' LDS copy rings fully fenced, for the
bit-identity race check). --sanitized also links _build/libmiattn_asan.so,
the C ABI layer under host AddressSanitizer + UndefinedBehaviorSanitizer.
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


# The race-detector variant (libmiattn_serial.so): the kernels with LDS copy
# rings, compiled with every ring copy fenced on both sides (see
# MIATTN_SERIAL_RINGS in csrc/common.hpp); every other object is shared.
SERIAL_OUT = os.path.join(HERE, "libmiattn_serial.so")
SERIAL_SOURCES = ["fwd_bf16.hip", "bwd.hip"]
SERIAL_DIR = os.path.join(BUILD_DIR, "serial")


def _compile(src: str, serial: bool = False) -> str:
    out_dir = SERIAL_DIR if serial else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS]
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    if serial:
        cmd += ["-DMIATTN_SERIAL_RINGS=1"]
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


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 4, verbose: bool = True) -> str:
    """Compile every source and link libmiattn.so, then the race-detector
    variant libmiattn_serial.so. Returns the path of libmiattn.so."""
    os.makedirs(SERIAL_DIR, exist_ok=True)
    jobs_list = [(s, False) for s in SOURCES] + [(s, True) for s in SERIAL_SOURCES]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda a: _compile(*a), jobs_list))
    main = objs[:len(SOURCES)]
    serial = dict(zip(SERIAL_SOURCES, objs[len(SOURCES):]))
    _link(main, OUT)
    _link([serial.get(s, o) for s, o in zip(SOURCES, main)], SERIAL_OUT)
    if verbose:
        print(f"built {OUT}")
        print(f"built {SERIAL_OUT}")
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
# layer (miattn.cpp: argument validation, dispatch), linked with the ordinary
# device objects. Only host code is instrumented: each sanitizer flag is
# passed to the host compilation alone. Run it with the clang runtime
# preloaded (asan_runtime()) and MIATTN_LIBRARY pointing at it.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan",
            "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_OUT = os.path.join(BUILD_DIR, "libmiattn_asan.so")


def asan_runtime() -> str:
    """The clang shared sanitizer runtime that the sanitized build links against."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("clang's shared ASan runtime was not found")
        path = hits[0]
    return path


def build_sanitized(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    dev_srcs = [s for s in SOURCES if s.endswith(".hip")]
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in dev_srcs]
    missing = [s for s, o in zip(dev_srcs, objs) if not os.path.exists(o)]
    if missing:
        with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            list(ex.map(_compile, missing))
    san_obj = os.path.join(BUILD_DIR, "miattn.cpp.asan.o")
    cmd = [hipcc(), *COMMON_FLAGS, *SANITIZE, "-g", "-c", os.path.join(CSRC, "miattn.cpp"),
           "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *SANITIZE, san_obj, *objs,
           "-o", SAN_OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--sanitized", action="store_true",
                    help="also build the host-sanitized C ABI library (_build/libmiattn_asan.so)")
    args = ap.parse_args()
    build(args.jobs)
    if args.sanitized:
        build_sanitized(args.jobs)


if __name__ == "__main__":
    main()
