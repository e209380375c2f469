"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle (oracle/kda_oracle.c) with tests/sanitize/oracle_driver.c:
  every entry point on small inputs in arrays of exactly the documented size,
  several threads, units without tokens, and the argument errors.
* The C ABI's argument checks (kda_api.cpp with the workspace layouts of
  kda_sizes.cpp), built host-only with launchers that launch nothing
  (tests/sanitize/api_stubs.cpp), driven by the whole of tests/test_abi.py.

A sanitizer finding aborts the run with a report, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    """Path of a sanitizer runtime gcc links against, or None."""
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or shutil.which("g++") is None or _runtime("libasan.so") is None,
    reason="gcc with AddressSanitizer is not available")


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L"] + SAN +
                   [os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    "-o", exe, "-lm", "-lpthread"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok" in res.stdout


def test_abi_checks_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not found")
    lib = str(tmp_path / "libkda_checks_san.so")
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC] + SAN +
                   [os.path.join(CSRC, "kda_api.cpp"), os.path.join(CSRC, "kda_sizes.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "api_stubs.cpp"), "-o", lib],
                   check=True)
    env = dict(os.environ)
    preload = [p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p]
    env["LD_PRELOAD"] = ":".join(preload)
    env["ASAN_OPTIONS"] = "detect_leaks=0"  # the interpreter's own allocations
    env["KDA_ABI_TEST_LIBRARY"] = lib
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
