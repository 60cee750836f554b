"""Build the HIP library (libvwl.so) and the measurement helper
(libvwl_bench.so: the read-only streaming reference kernel) for gfx950 with
hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libvwl.so")
BENCH_LIB = os.path.join(LIBDIR, "libvwl_bench.so")
BENCH_SOURCES = ["stream_ref.hip"]
SOURCES = ["asym_ab.hip", "asym_a.hip", "asym_tb.hip", "pair_pass.hip", "lmhead.hip", "rapid.hip",
           "vwl_api.cpp"]
HEADERS = ["asym_kernels.hpp", "vwl_device.hpp", "vwl_internal.hpp", "vwl_stage.hpp"]

ARCH = os.environ.get("VWL_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are disabled for every HIP translation unit.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall"]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-6000:]))


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr[-6000:])
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)


def build(verbose: bool = False) -> str:
    """Compile every source and link libvwl.so and libvwl_bench.so (always
    rebuilds)."""
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    objs = [os.path.join(LIBDIR, os.path.splitext(s)[0] + ".o") for s in srcs]
    with ThreadPoolExecutor(len(srcs)) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print("built", LIB, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
