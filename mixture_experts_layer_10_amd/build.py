"""Build the HIP library in-tree: mixture_experts_layer_10_amd/_lib/libmoe_mi355x.so (gfx950 only).

    python -m mixture_experts_layer_10_amd.build [--jobs N]

Every .hip file under csrc/ is compiled separately with hipcc (parallel), then linked into one
shared library exporting the C ABI declared in include/moe.h. probe/ceilings.hip (the benchmark's
measured read and matrix-core ceilings, not part of the ABI) becomes _lib/libmoe_probe.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(OUT_DIR, LIB_NAME)
PROBE_SRC = os.path.join(PKG, "probe", "ceilings.hip")
PROBE_PATH = os.path.join(OUT_DIR, "libmoe_probe.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    # the measured-ceiling probes of the benchmark: a small library of their own
    ptmp = PROBE_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-o", ptmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(ptmp, PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources, and {PROBE_PATH}")
    return LIB_PATH


# Host AddressSanitizer build for the CPU tests: the same sources with the host code instrumented
# (device code unchanged), linked against the shared sanitizer runtime, which the test process
# preloads. It stays under _build/ and is never loaded by the product path.
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libmoe_mi355x_hostasan.so")
ASAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
ASAN_LINK_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -shared-libasan".split()


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm clang."""
    for clang in ("/opt/rocm/llvm/bin/clang", shutil.which("amdclang") or ""):
        if clang and os.path.exists(clang):
            r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("AddressSanitizer runtime not found")


def _compile_asan(src: str) -> str:
    obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
    flags = [f for f in HIP_FLAGS if f != "-O3"]
    cmd = [hipcc(), *flags, "-O1", *ASAN_HOST_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_host_asan(jobs: int | None = None) -> str:
    """Builds ASAN_LIB_PATH unless it is newer than every source and header."""
    srcs = sources()
    inc = os.path.join(ROOT, "include")
    deps = srcs + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(inc, f) for f in os.listdir(inc)]
    if os.path.exists(ASAN_LIB_PATH) and os.path.getmtime(ASAN_LIB_PATH) > max(os.path.getmtime(d) for d in deps):
        return ASAN_LIB_PATH
    os.makedirs(ASAN_DIR, exist_ok=True)
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile_asan, srcs))
    tmp = ASAN_LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_LINK_FLAGS, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB_PATH)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
