"""GPU parity of the many-column path (Q4_K, n >= 6 activation columns, int8
matrix cores) through the C ABI: against the oracle within the stated
tolerance for every row and column, at shapes with ragged row and column
tiles, at the FFN-down workload with 64 columns (sampled rows), with the
epilogue's scale and bias, and the argument checks of the path."""
import numpy as np
import pytest

import oracle
from gpu_helpers import announce, assert_close, dev, gpu_quantize, host
from quantized_decode_gemv_quantize_amd import binding as B
from quantized_decode_gemv_quantize_amd import synth

pytestmark = pytest.mark.gpu

Q4_K = B.Q4_K


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _nan(rows, M):
    import torch
    return torch.full((rows, M), float("nan"), dtype=torch.float32, device="cuda:0")


# The launch picks its tile and wave count from the grid size; on a 256-CU
# part the last four shapes take 2x2 tiles with 4 waves, 2x1 with 4, 2x1
# with 8 and 1x1 with 4 (the others 1x1 with 8; the workload test 2x2 with 8).
SHAPES = [(1, 256, 9), (37, 512, 16), (300, 2304, 17), (1000, 4096, 33), (129, 14336, 64),
          (65, 16384, 100), (33, 768, 256), (17, 1280, 31),
          (9000, 256, 32), (9000, 512, 16), (8192, 256, 9), (5000, 256, 16),
          (300, 2304, 6), (129, 14336, 7), (1000, 4096, 8)]


@pytest.mark.parametrize("M,K,n", SHAPES, ids=[f"{m}x{k}-n{n}" for m, k, n in SHAPES])
def test_many_columns_parity(O, M, K, n):
    announce(f"mmvq many columns q4_k M={M} K={K} n={n}")
    rng = np.random.default_rng(M + K + n)
    W = synth.weights(Q4_K, M, K, rng)
    x = synth.activations(K, n, rng)
    yd = gpu_quantize(x)
    y = O.quantize_q8_1(x)
    assert np.array_equal(host(yd), y)
    out = _nan(n, M)
    B.mmvq(dev(W), Q4_K, M, K, yd, n, out)
    ref, mag, _ = O.mmvq(W, Q4_K, M, K, y, n)
    assert_close(host(out), ref, mag, f"many columns {M}x{K} n={n}")


def test_many_columns_workload(O):
    """FFN-down shape (4096 x 14336) with 64 columns, the launch the
    benchmark times; every row and column against the oracle."""
    wl = synth.BY_NAME["q4_k_4096x14336"]
    n = 64
    announce(f"mmvq many columns workload n={n}")
    rng = np.random.default_rng(4242)
    W = synth.make(wl, 1)["W"]
    x = synth.activations(wl.K, n, rng)
    yd = gpu_quantize(x)
    y = O.quantize_q8_1(x)
    out = _nan(n, wl.M)
    B.mmvq(dev(W), Q4_K, wl.M, wl.K, yd, n, out)
    ref, mag = O.mmvq_threaded(W, Q4_K, wl.M, wl.K, y, n)
    assert_close(host(out), ref, mag, "many columns workload")


def test_many_columns_epilogue(O):
    """mmvq_ex without a gate: scale and bias rows on the many-column path."""
    M, K, n = 300, 2048, 40
    announce(f"mmvq_ex many columns M={M} K={K} n={n}")
    rng = np.random.default_rng(77)
    W = synth.weights(Q4_K, M, K, rng)
    x = synth.activations(K, n, rng)
    bias = rng.standard_normal(M).astype(np.float32)
    scale = np.float32([0.75])
    bd, sd = dev(bias), dev(scale)
    out = _nan(n, M)
    B.mmvq_ex(dev(W), None, Q4_K, M, K, gpu_quantize(x), None, 0, n, B.epilogue(up_bias=bd, up_scale=sd), out)
    y = O.quantize_q8_1(x)
    ref = O.mmvq_ex(W, None, Q4_K, M, K, y, n, dict(up_bias=bias.astype(np.float64), up_scale=[0.75]))
    _, mag, _ = O.mmvq(W, Q4_K, M, K, y, n)
    # scale then bias: the product's bound scaled, plus the fp32 roundings of both steps
    tol = 0.75 * (1e-5 * mag + 1e-6) + 2.0 ** -22 * (np.abs(ref) + np.abs(bias)) + 1e-6
    got = host(out).astype(np.float64)
    bad = ~(np.abs(got - ref) <= tol)
    assert not bad.any(), np.argwhere(bad)[0]


def test_many_columns_quantize_bitexact(O):
    announce("quantize n=100")
    rng = np.random.default_rng(3)
    x = synth.activations(1024, 100, rng, 1030)
    assert np.array_equal(host(gpu_quantize(x, 1024)), O.quantize_q8_1(x, 1024))


def test_many_columns_argument_checks():
    import torch
    announce("many columns abi errors")
    W = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0")
    y = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0")
    out = torch.zeros(1 << 16, dtype=torch.float32, device="cuda:0")
    L = B.lib()
    s = torch.cuda.current_stream().cuda_stream
    p, q, o = W.data_ptr(), y.data_ptr(), out.data_ptr()
    assert L.mmvq(p, Q4_K, 1, 256, q, 257, o, s) == B.ERR_SHAPE
    assert L.mmvq(p, B.Q4_0, 1, 256, q, 9, o, s) == B.ERR_SHAPE
    assert L.mmvq(p, 7, 1, 256, q, 9, o, s) == B.ERR_TYPE
    assert L.mmvq(p, Q4_K, 1, 200, q, 9, o, s) == B.ERR_SHAPE
    assert L.mmvq(p + 4, Q4_K, 1, 256, q, 9, o, s) == B.ERR_ALIGN
    assert L.mmvq_glu(p, p, Q4_K, 1, 256, q, 9, 1, o, s) == B.ERR_SHAPE
    assert L.mmvq_f32(p, Q4_K, 1, 256, o, 9, 256, o, s) == B.ERR_SHAPE
    torch.cuda.synchronize()
