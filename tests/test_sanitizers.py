"""CPU-side safety layers: the oracle and the host models of the kernels'
addressing, built with the address and undefined-behaviour sanitizers
(host code only: the oracle is plain C, the host models compile the kernels'
format and planning headers for the CPU) and run on reduced case sets. Any
out-of-bounds access, use after free, signed overflow or invalid shift
aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "quantized_decode_gemv_quantize_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host_model")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _tool(*cands):
    for c in cands:
        p = c if os.path.isabs(c) else shutil.which(c)
        if p and os.path.exists(p):
            return p
    pytest.skip(f"none of {cands} available")


def _run(exe, *args, timeout=300):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=timeout, env=env)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-4000:]
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_drive"
    subprocess.check_call([_tool("gcc"), "-std=c11", "-ffp-contract=off", *SAN, "-o", str(exe),
                           os.path.join(HOST, "oracle_drive.c"), os.path.join(ROOT, "oracle", "mmvq_oracle.c"),
                           "-lm"])
    assert "ok: 0 failure(s)" in _run(exe)


def test_host_models_under_sanitizers(tmp_path):
    cxx = _tool("/opt/rocm/llvm/bin/clang++", "clang++")
    bounds = tmp_path / "bounds"
    subprocess.check_call([cxx, "-std=c++17", *SAN, "-DQMV_HOST_MODEL", "-I", INC, "-o", str(bounds),
                           os.path.join(HOST, "bounds.cpp")])
    assert "0 failing case(s)" in _run(bounds, "small")
    q8 = tmp_path / "q8_fast"
    subprocess.check_call([cxx, "-std=c++17", "-ffp-contract=off", *SAN, "-DQMV_HOST_MODEL", "-I", INC, "-o",
                           str(q8), os.path.join(HOST, "q8_fast.cpp")])
    assert " 0 mismatches" in _run(q8, "20000")
