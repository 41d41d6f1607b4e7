"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/hc_oracle.c) is built with gcc, OpenMP on, and
  tests/sanitize/oracle_driver.c runs every one of its functions on small
  seeded inputs in buffers of exactly the documented sizes.
* The C-ABI's checking layer (csrc/hc_api.hip: argument checks, size
  queries, dispatch) is built with hipcc, the sanitizers on its host code
  only, and linked against libhc.so for the kernel launchers, which the
  checks never reach; tests/sanitize/abi_driver.cpp drives every entry
  point of include/hc.h along its error paths and size queries.

Both drivers exit 0 only when every call returned as documented; a
sanitizer report makes them fail.
"""
import os
import shutil
import subprocess

import pytest

import hyper_connection_residual_02_amd as hcl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    out = r.stdout + r.stderr
    assert r.returncode == 0, "%s failed (%d):\n%s" % (cmd[0], r.returncode, out[-4000:])
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "hc_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    out = _run([exe], env=ENV)
    assert "ok" in out and "ERROR" not in out and "runtime error" not in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_checks_under_sanitizers(tmp_path):
    if not os.path.exists(hcl.lib_path()):
        import hyper_connection_residual_02_amd.build as b
        b.build(verbose=False)
    csrc = os.path.join(ROOT, "hyper_connection_residual_02_amd", "csrc")
    # sanitizers on the host code only: each -fsanitize= follows -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    api_o, drv_o, exe = str(tmp_path / "hc_api.o"), str(tmp_path / "driver.o"), str(tmp_path / "abi_driver")
    _run([HIPCC, *common, *host_san, "-c", os.path.join(csrc, "hc_api.hip"), "-o", api_o])
    _run([HIPCC, *common, *host_san, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv_o])
    libdir = os.path.dirname(hcl.lib_path())
    _run([HIPCC, "--offload-arch=gfx950", "-fno-gpu-sanitize", "-fsanitize=address", "-fsanitize=undefined",
          api_o, drv_o, hcl.lib_path(), "-Wl,-rpath," + libdir, "-o", exe])
    out = _run([exe], env=ENV)
    assert "ok" in out and "ERROR" not in out and "runtime error" not in out, out
