"""The host C/C++ code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the fp64 oracle (oracle/oracle.c) and the library's host
packers and quantizers (csrc/pack.cpp, csrc/quant.cpp, host code built by
ROCm's clang++ with no GPU target), each linked into a driver of its own that runs every entry point on small ragged shapes.  The
two are built apart: the oracle and the library share no code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")

# The host C++ uses _Float16 (IEEE binary16 conversions), which this image's
# g++ does not accept on x86; ROCm's clang++ builds it as plain host code.
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _build_and_run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    cmd = ["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"]
    assert "oracle checks passed" in _build_and_run(cmd, exe, tmp_path)


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="needs ROCm's clang++")
def test_host_packers_and_quantizers_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    csrc = os.path.join(ROOT, "speculative_verify_amd", "csrc")
    cmd = [CLANGXX, "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), os.path.join(csrc, "pack.cpp"),
           os.path.join(csrc, "quant.cpp"), "-o", exe, "-lpthread"]
    assert "host checks passed" in _build_and_run(cmd, exe, tmp_path)
