"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/sanitize/oracle_driver.c exercises every oracle entry point;
tests/sanitize/host_driver.cpp exercises the library's host side (format
set-up and validation, the decode planner, every entry point's argument
checks), which runs no GPU code.  Both are built here with the sanitizers on
the host code only and must run clean.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    return log


def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        subprocess.run(["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "oracle"),
                        os.path.join(SAN, "oracle_driver.c"),
                        os.path.join(ROOT, "oracle", "hkv_oracle.c"), "-o", exe, "-lm",
                        "-lpthread"], check=True)
        assert "oracle driver: ok" in _run(exe)


@pytest.mark.skipif(shutil.which("hipcc") is None and
                    not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not found")
def test_host_code_under_asan_ubsan():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    csrc = os.path.join(ROOT, "decode_attention_amd", "csrc")
    srcs = sorted(os.path.join(csrc, n) for n in os.listdir(csrc) if n.endswith(".hip"))
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_driver")
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                        "-ffp-contract=off",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-I", os.path.join(ROOT, "include"), "-I", csrc,
                        os.path.join(SAN, "host_driver.cpp"), *srcs, "-o", exe],
                       check=True, capture_output=True)
        assert "host driver: ok" in _run(exe)
