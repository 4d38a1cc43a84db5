"""Sanitizer builds of the host code (no GPU): the CPU oracle, and the C-ABI's
argument checks and dispatch with the kernel launchers replaced by stand-ins.

Both are compiled with AddressSanitizer and UndefinedBehaviorSanitizer (no
recovery, so any report fails the run) and exercised by the drivers in
tests/sanitize/: every oracle function on small inputs, and every entry point
of include/ulysses.h with accepted and rejected arguments, including sizes
whose products overflow 64 bits.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_checks"
    _run(["gcc", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", *SAN,
          os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-o", str(exe), "-lm"])
    r = _run([str(exe)], env=dict(ENV, OMP_NUM_THREADS="3"))
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not found")
def test_abi_checks_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_checks"
    _run(["g++", "-std=c++17", *SAN, "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
          "-x", "c++", os.path.join(ROOT, "sequence_long_context_amd", "csrc", "api.hip"),
          "-x", "c++", os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cc"),
          os.path.join(ROOT, "tests", "sanitize", "abi_checks.cc"), "-o", str(exe)])
    r = _run([str(exe)], env=ENV)
    assert "0 failures" in r.stdout
