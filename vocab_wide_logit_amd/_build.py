"""Build the HIP library (libvwl.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libvwl.so")
SOURCES = ["asym_ab.hip", "asym_a.hip", "asym_tb.hip", "pair_pass.hip", "lmhead.hip", "rapid.hip",
           "vwl_api.cpp"]
HEADERS = ["asym_kernels.hpp", "vwl_device.hpp", "vwl_internal.hpp"]

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


def build(verbose: bool = False) -> str:
    """Compile every source and link libvwl.so (always rebuilds)."""
    os.makedirs(LIBDIR, exist_ok=True)
    objs = [os.path.join(LIBDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr[-6000:])
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
