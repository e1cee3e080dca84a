"""Build libpkv.so (HIP kernels for gfx950 + host C++), in-tree.

    python -m paged_kv_cache_indirected_amd.build

Host translation units are compiled by g++, HIP ones by hipcc for gfx950
only, then linked with hipcc into the package directory.  The same sources
are built a second time with PKV_DEBUG defined into libpkv_debug.so: every
call that enqueues device work then synchronises and reports the device
preconditions the kernels found violated (the binding loads it when the
environment sets PKV_DEBUG=1).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
DEBUG_LIB = os.path.join(PKG, "libpkv_debug.so")
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")   # measurement probes, loaded by the benchmark only
OBJ = os.path.join(ROOT, "_build", "pkv")
OBJ_DEBUG = os.path.join(ROOT, "_build", "pkv_debug")

HOST_SRC = ["errors.cpp", "pool.cpp", "sched.cpp", "api.cpp"]
HIP_SRC = ["append.hip", "copy.hip", "debug.hip", "decode.hip", "prefill.hip", "side_stream.hip"]

ARCH = "gfx950"
# Packed fp32 vector ops are switched off for all device code.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-I" + INCLUDE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ_DEBUG, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for obj, extra in ((OBJ, []), (OBJ_DEBUG, ["-DPKV_DEBUG"])):
        for s in HOST_SRC:
            jobs.append(["g++", *HOST_FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o",
                         os.path.join(obj, s + ".o")])
        for s in HIP_SRC:
            jobs.append([hipcc, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o",
                         os.path.join(obj, s + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    for obj, lib in ((OBJ, LIB), (OBJ_DEBUG, DEBUG_LIB)):
        tmp = lib + ".tmp"
        objs = [os.path.join(obj, s + ".o") for s in HOST_SRC + HIP_SRC]
        # -z defs: a symbol left undefined (e.g. a kernel whose host stub was
        # not emitted) fails the build instead of the library's first load.
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o",
              tmp])
        os.replace(tmp, lib)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, *HIP_FLAGS, "-shared", os.path.join(CSRC, "probe.hip"), "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
