"""Build ``libmmvq.so`` (the HIP library behind ``include/mmvq.h``) for gfx950.

Run ``python -m quantized_decode_gemv_quantize_amd.build`` or call
``build()``. Every call recompiles. The library is written in-tree, next to
this file, so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmmvq.so")
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"

# Longest first: the expert-indexed Q4_K kernels sit in units of their own so
# the fp32 Q4_K unit does not set the build time alone.
SOURCES = ["kernels_q4_k_f32.hip", "kernels_q4_k_f32_id.hip", "kernels_q4_k.hip", "kernels_q4_k_id.hip",
           "kernels_q6_k_f32.hip", "kernels_q6_k.hip", "kernels_q4_0_f32.hip", "kernels_q8_0_f32.hip",
           "kernels_q4_0.hip", "kernels_q8_0.hip", "kernels_q5_k_f32.hip", "kernels_q5_k.hip",
           "kernels_q4_1_f32.hip", "kernels_q5_0_f32.hip", "kernels_q5_1_f32.hip", "kernels_q4_1.hip",
           "kernels_q5_0.hip", "kernels_q5_1.hip", "kernels_mmq.hip", "kernels_mmq_f32.hip", "api.hip", "quantize.hip",
           "probe.hip"]

# Packed fp32 VALU instructions stay disabled (hipcc forms them from plain
# float code otherwise); fp32 division is correctly rounded and fp32
# denormals are kept, which the q8_1 step relies on to match its definition.
# No implicit fp contraction: every fused multiply-add is an explicit fmaf in
# the source, so each kernel instantiation (q8_1 or fp32 activations, any
# row count) rounds the same operations the same way.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


# Per-source flags. The many-column kernel keeps its matrix-core results in
# ordinary vector registers (the scale arithmetic reads every result; in
# accumulation registers each value would first be copied out).
SOURCE_FLAGS = {
    "kernels_mmq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernels_mmq_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(extra_flags: list[str] | None = None, jobs: int | None = None, out: str = LIB) -> str:
    """Compile all sources and link the shared library; returns its path."""
    extra = list(extra_flags or [])
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
