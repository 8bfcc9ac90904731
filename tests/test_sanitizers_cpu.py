"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/kda_oracle.c, with OpenMP) driven by
  tests/sanitize/oracle_driver.c: packed sequences with empty ones, NULL and
  aliased states, rejected arguments.
* The C ABI's host side (csrc/kda_api.cpp) driven by
  tests/sanitize/abi_driver.cpp with stub launchers: every entry point's
  checks, out-of-range enum values, and valid calls into launch sequencing.

Both build as standalone host executables (no GPU code, no HIP runtime
calls) and must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]
CLANG = Path("/opt/rocm/llvm/bin/clang++")


def _run(cmd, tmp, exe):
    subprocess.run(cmd, check=True, cwd=tmp, capture_output=True, text=True, timeout=240)
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], cwd=tmp, capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_driver"
    out = _run(["gcc", "-std=c11", "-fopenmp", *SAN, "-Wall", "-Wextra", "-o", str(exe),
                str(ROOT / "oracle" / "kda_oracle.c"),
                str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-lm"], tmp_path, exe)
    assert "oracle driver ok" in out


def test_abi_host_side_under_sanitizers(tmp_path):
    if not CLANG.exists() or not Path("/opt/rocm/include/hip/hip_runtime.h").exists():
        pytest.skip("ROCm clang++ or HIP headers not available")
    exe = tmp_path / "abi_driver"
    out = _run([str(CLANG), "-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                "-I/opt/rocm/include", f"-I{ROOT / 'include'}", *SAN, "-o", str(exe),
                str(ROOT / "gated_delta_rule_50_amd" / "csrc" / "kda_api.cpp"),
                str(ROOT / "tests" / "sanitize" / "abi_driver.cpp")], tmp_path, exe)
    assert "abi driver ok" in out
