"""Build the native library ``libgcs.so`` in-tree for gfx950.

Host-only builder sources are compiled with g++; the device engine with hipcc
for gfx950 only; hipcc links both into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libgcs.so")
OBJ = os.path.join(PKG, "_build")

HOST_SOURCES = ["builder.cpp", "repair.cpp", "repair_rounds.cpp", "serialize.cpp"]
DEVICE_SOURCES = ["sweep.hip", "build_gpu.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 instructions are disabled for all device code
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter", "-pthread"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {os.path.basename(cmd[-1])}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    objs = []
    for s in HOST_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        objs.append(o)
        jobs.append(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", o, os.path.join(CSRC, s)])
    for s in DEVICE_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        objs.append(o)
        jobs.append([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", o, os.path.join(CSRC, s)])
    with ThreadPoolExecutor(max_workers=4) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout + r.stderr)
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-pthread"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
