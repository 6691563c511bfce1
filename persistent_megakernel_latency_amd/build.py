"""Builds libwpk.so (the C ABI + gfx950 kernels) and the microbenchmark, in-tree.

    python -m persistent_megakernel_latency_amd.build

Every HIP translation unit is compiled with hipcc for gfx950 only, with packed
fp32 instructions disabled.  The host-only C++ (builder, host executors) is
compiled by the same hipcc as plain C++.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwpk.so")
MICROBENCH = os.path.join(HERE, "wpk_microbench")

ARCH = "gfx950"
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I/opt/rocm/include"]

DEVICE_SOURCES = ["megakernel.hip", "persist.hip", "prefill.hip"]
HOST_SOURCES = ["capi.cpp", "builder.cpp", "host_exec.cpp", "planner.cpp", "prefill_builder.cpp", "prefill_capi.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    jobs = []
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        jobs.append(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        jobs.append(["/opt/rocm/llvm/bin/clang++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=4) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg:
                print(msg)
    tmp = LIB + ".tmp"
    _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"])
    os.replace(tmp, LIB)
    tmp = MICROBENCH + ".tmp"
    _run(["hipcc", *HIP_FLAGS, os.path.join(CSRC, "microbench.hip"), "-o", tmp])
    os.replace(tmp, MICROBENCH)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
