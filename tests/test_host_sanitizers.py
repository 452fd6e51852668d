"""Host code under the address and undefined-behaviour sanitizers (no GPU needed).

- The C oracle, every entry point on small seeded inputs (tests/sanitize/oracle_driver.c, built
  with gcc).
- The library's host side: kvq_host.cpp rebuilt with the sanitizers on its host code and linked
  with the kernel objects of the last build, driven through the C ABI over argument refusals,
  tables, record sizes, workspace sizes and the cache bookkeeping (tests/sanitize/
  host_driver.cpp). Nothing reaches a device: every call returns before a launch.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OBJ = os.path.join(ROOT, "kv_cache_compression_vector_amd", "_obj")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers for host code only: each flag follows -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd, timeout=300):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-D_GNU_SOURCE", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"], ROOT)
    r = _run([exe], ROOT)
    assert "oracle driver ok" in r.stdout


def test_library_host_code_under_address_and_ub_sanitizers(tmp_path):
    objs = sorted(os.path.join(OBJ, f) for f in os.listdir(OBJ)
                  if f.endswith(".o") and f != "kvq_host.o") if os.path.isdir(OBJ) else []
    if not os.path.exists(HIPCC) or len(objs) < 5:
        pytest.skip("needs hipcc and the kernel objects of a library build (__graft_entry__.build())")
    host_o, drv_o, exe = (str(tmp_path / n) for n in ("host_san.o", "driver.o", "host_driver"))
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-rdc"] + HOST_SAN +
         ["-c", os.path.join(ROOT, "kv_cache_compression_vector_amd", "csrc", "kvq_host.cpp"),
          "-o", host_o], ROOT)
    _run([HIPCC, "-O1", "-g", "-std=c++17"] + HOST_SAN +
         ["-c", os.path.join(SAN, "host_driver.cpp"), "-o", drv_o], ROOT)
    _run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN + [drv_o, host_o] + objs + ["-o", exe], ROOT)
    r = _run([exe], ROOT, timeout=120)
    assert "host driver ok" in r.stdout
