"""Host-side checks of the benchmark's bookkeeping (no GPU): which form a
profiled kernel belongs to, the algorithmic bytes the roofline divides by,
and the refusal of multi-GPU runs."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_decode_gemv_quantize_amd import synth  # noqa: E402


@pytest.mark.parametrize("name,form", [
    ("void qmv::mmvq_rows_kernel<qmv::Q6K, 1, 8, 1, 1, true, 1, 0, false>(qmv::RowArgs)", "fused"),
    ("void qmv::mmvq_rows_kernel<qmv::Q6K, 1, 8, 1, 1, false, 1, 0, false>(qmv::RowArgs)", "gemv"),
    ("void qmv::mmvq_rows1_kernel<qmv::Q4K, 16, 4, true, 0>(qmv::RowArgs)", "fused"),
    ("void qmv::mmvq_rows1_kernel<qmv::Q4K, 4, 0, false, 0>(qmv::RowArgs)", "gemv"),
    ("void qmv::mmq_kernel<qmv::Q4K, 2, 2, 4, 1, false>(qmv::MmqArgs)", "gemv"),
    ("void qmv::mmq_kernel<qmv::Q4K, 2, 1, 4, 1, true>(qmv::MmqArgs)", "fused"),
    ("qmv::quantize_q8_1_kernel(float const*, unsigned char*, long, long, long)", "quantize"),
    ("qmv::read_probe_kernel(unsigned char const*, long, unsigned int*)", "probe"),
    ("void qmv::mmvq_id_kernel<qmv::Q4K2, 8, 1, 2, false, false>(qmv::RowArgs)", "id"),
    ("void qmv::mmvq_id_kernel<qmv::Q4K2, 32, 1, 2, true, false>(qmv::RowArgs)", "id_fused"),
    ("__amd_rocclr_copyBuffer", None),
])
def test_kernel_form(name, form):
    assert bench.kernel_form(name) == form


def test_kernel_form_shared_expert_slice():
    name = "void qmv::mmvq_id_kernel<qmv::Q4K2, 8, 1, 2, false, false>(qmv::RowArgs)"
    assert bench.kernel_form(name, grid_y=9, n_experts=8) == "id_shared"
    assert bench.kernel_form(name, grid_y=8, n_experts=8) == "id"


def test_algorithmic_bytes_headline():
    """Q4_K 4096x14336, one column: 33,030,144 weight bytes; q8_1 column
    448 x 36 = 16,128 B; fp32 column 14336 x 4 = 57,344 B; outputs 16,384 B."""
    wl = synth.BY_NAME["q4_k_4096x14336"]
    assert wl.weight_bytes == 33_030_144
    assert bench.algorithmic_bytes(wl, 1) == 33_030_144 + 16_128 + 16_384
    assert bench.fused_bytes(wl, 1) == 33_030_144 + 57_344 + 16_384
    assert bench.algorithmic_bytes(wl, 128) == 33_030_144 + 128 * 16_128 + 128 * 16_384


def test_multi_gpu_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""
