"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU work).

* The fp64 oracle (oracle/oracle.c) under both sanitizers, driven by tests/sanitize/oracle_driver.c:
  every routine on small seeded inputs, optional arguments on and off, ragged shapes.
* The library's host code (csrc/*.hip built with the sanitizers on the host side only; the
  device code is compiled as usual and never launched), driven by tests/sanitize/abi_driver.c:
  every workspace query over a sweep of shapes and the rejected-argument path of every entry
  point. A sanitizer report aborts the driver with a non-zero status."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_37_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizer options of the host compiler pass only (each after -Xarch_host)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11"] + GCC_SAN +
         [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], timeout=120)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I" + INCLUDE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC] + flags + ["-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "-x", "c", "-O1", "-g", "-std=c11", "-I" + INCLUDE] + HOST_SAN +
         ["-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN + [drv] + objs + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")   # the HIP runtime keeps its own allocations
    r = _run([exe], timeout=300, env=env)
    assert "abi driver ok" in r.stdout
