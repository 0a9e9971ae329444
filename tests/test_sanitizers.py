"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

- oracle/moe_oracle.c with tests/sanitize/oracle_driver.c (gcc): every
  oracle entry point on small seeded layers (fp32 and bf16, drops,
  capacity 0, k = E, T = 1, router bias, residual), leak detection on.
- libmoe.so with its host code sanitized (hipcc, the sanitizer flags passed
  to the host compilation only) and tests/sanitize/host_driver.cpp (clang++):
  argument validation of every entry point, workspace sizes over a grid of
  shapes, the expert-cache policy over random step sequences and the
  host-side permutation check on valid and corrupted permutations. No call
  reaches the GPU.
Each run must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, report
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-std=c99", "-Wall",
                    "-Werror", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], check=True)
    out = _run(exe)
    assert out.count("loss") == 7


CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") and os.path.exists(CLANG)),
                    reason="no ROCm compilers")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from top_routing_expert_topk_amd import build as hip_build
    lib = hip_build.build_host_sanitized(str(tmp_path / "libmoe_san.so"))
    exe = str(tmp_path / "host_san")
    subprocess.run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(SAN, "host_driver.cpp"), lib, f"-Wl,-rpath,{tmp_path}",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    assert "all expectations met" in _run(exe)
