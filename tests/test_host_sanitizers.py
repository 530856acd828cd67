"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C driver ``tests/sanitize/host_checks.c`` calls every entry point with
arguments its host checks must reject (and with nothing to do), and checks
the status codes. The library is rebuilt with both sanitizers on its host
code only (device code is compiled as usual); every call ends before any HIP
runtime call, so no GPU is needed. Any sanitizer report fails the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_host_checks_clean_under_sanitizers(tmp_path):
    lib = tmp_path / "libgg_san.so"
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-o", str(lib),
             os.path.join(ROOT, "moe_ragged_grouped_amd", "csrc", "grouped_gemm.hip")]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "host_checks"
    link = [CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "host_checks.c"),
            "-L", str(tmp_path), "-lgg_san", "-Wl,-rpath," + str(tmp_path), "-o", str(exe)]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # the HIP runtime itself is not instrumented; its allocations at load time
    # are not this library's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert "host checks: 0 failure(s)" in r.stdout
