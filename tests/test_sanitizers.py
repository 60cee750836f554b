"""The fp64 oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (no GPU needed).

* ``tests/sanitize/oracle_harness.c`` drives every oracle entry point on
  small seeded inputs, both dtypes, the degenerate shapes and bad ids,
  built together with ``oracle/vwl_oracle.c`` by gcc.
* ``tests/sanitize/host_harness.cpp`` drives the library's host side:
  status strings for any int, every workspace-size query over ordinary and
  extreme shapes, and the argument checks of the entry points (each case
  returns before any device work).  ``vwl_api.cpp`` is built with the
  sanitizers on its host pass only, and ``host_stubs.cpp`` stands in for the
  kernel launchers (a launch reaching one aborts the run).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_h")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(HERE, "oracle_harness.c"),
          os.path.join(ROOT, "oracle", "vwl_oracle.c"), "-lm"])
    r = _run([exe], env=SAN_ENV)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_asan_ubsan(tmp_path):
    # sanitizers on the host pass only (each flag behind -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    comp = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
            "-I", os.path.join(ROOT, "include")] + san
    objs = []
    for src in (os.path.join(ROOT, "vocab_wide_logit_amd", "csrc", "vwl_api.cpp"),
                os.path.join(HERE, "host_stubs.cpp"), os.path.join(HERE, "host_harness.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(comp + ["-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_h")
    _run([HIPCC, "--offload-arch=gfx950"] + san[:4] + ["-o", exe] + objs)
    r = _run([exe], env=SAN_ENV)
    assert "all checks passed" in r.stdout
