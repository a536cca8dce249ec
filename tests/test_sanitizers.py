"""Host code under the host compiler's address and undefined-behaviour
sanitizers (no GPU): the C ABI's validation, workspace carving and dispatch
(convrot_api.cpp against stand-in launchers and a host-only stand-in for the
HIP header, tests/sanitize/), and the CPU oracle (convrot_oracle.c), each
driven through its entry points on valid and invalid arguments.  A sanitizer
report makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "int8_hadamard_rotated_amd", "csrc")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs the host gcc toolchain")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    run(["g++", "-std=c++17", *FLAGS, "-I", SAN, "-I", CSRC,
         os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "stubs.cpp"),
         os.path.join(CSRC, "convrot_api.cpp"), "-o", exe])
    out = run([exe], env=ENV).stdout
    assert "abi ok" in out


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", *FLAGS, "-ffp-contract=off", "-fopenmp",
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "convrot_oracle.c"),
         "-o", exe, "-lm"])
    out = run([exe], env=dict(ENV, OMP_NUM_THREADS="2")).stdout
    assert "oracle ok" in out
