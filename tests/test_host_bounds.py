"""Every memory access of the kernels, checked on the CPU.

Builds tests/host_model/bounds.cpp against the library's own format and
launch-planning headers with QMV_HOST_MODEL (loads become bounds-checked host
reads) and runs it over many shapes, including the benchmark workloads: every
load of every lane must stay inside its buffer with the alignment its device
load needs, and every output row must be stored exactly once."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_model", "bounds.cpp")
INC = os.path.join(ROOT, "quantized_decode_gemv_quantize_amd", "csrc")


def _clang():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("clang++ (host) not available")


def test_kernel_accesses_in_bounds(tmp_path):
    exe = tmp_path / "bounds"
    subprocess.check_call([_clang(), "-std=c++17", "-O2", "-DQMV_HOST_MODEL", "-I", INC, "-o", str(exe),
                           SRC])
    res = subprocess.run([str(exe), "full"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    assert "0 failing case(s)" in res.stdout


def test_q8_fast_quantizer_exact(tmp_path):
    """The quantizer's reciprocal fast path with exact fallback (q8.hpp)
    gives roundf(x/d) for every value: random blocks at all scales and values
    placed within 8 ulps of every code boundary, on the host."""
    exe = tmp_path / "q8_fast"
    subprocess.check_call([_clang(), "-std=c++17", "-O2", "-ffp-contract=off", "-DQMV_HOST_MODEL", "-I", INC,
                           "-o", str(exe), os.path.join(ROOT, "tests", "host_model", "q8_fast.cpp")])
    res = subprocess.run([str(exe), "400000"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    assert " 0 mismatches" in res.stdout
