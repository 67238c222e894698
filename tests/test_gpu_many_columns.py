"""GPU parity of the many-column path (more than the row kernels' columns,
int8 matrix cores; every weight format with q8_1 activations, with or
without a gate) through the C ABI: against the oracle within the stated tolerance for
every row and column, at shapes with ragged row and column tiles, at the
FFN-down and LM-head workloads, with the epilogue's scale and bias; the
fp32-activation and gate/up forms beyond 8 columns, and the forms that run
as column groups through the row kernels (K not a multiple of 256); and the
argument checks of the path."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TNAME, announce, assert_close, dev, glu_tolerance, gpu_quantize, host
from quantized_decode_gemv_quantize_amd import binding as B
from quantized_decode_gemv_quantize_amd import synth

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = B.Q4_0, B.Q8_0, B.Q4_K, B.Q6_K


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
# part the shapes with 9000 / 8192 / 5000 rows take 2x2 tiles with 4 waves,
# 2x1 with 4, 2x1 with 8 and 1x1 with 4 (the others 1x1 with 8). Q6_K rows
# are only 2-byte aligned: their super-blocks sit at every even offset from
# a 16-byte boundary across rows and steps. Q4_K takes the path from 6
# columns, the other formats from 9.
SHAPES = [(1, 256, 9), (37, 512, 16), (300, 2304, 17), (1000, 4096, 33), (129, 14336, 64),
          (65, 16384, 100), (33, 768, 256), (17, 1280, 31),
          (9000, 256, 32), (9000, 512, 16), (8192, 256, 9), (5000, 256, 16)]
CASES = [(t, M, K, n) for t in (Q4_K, Q6_K, Q4_0, Q8_0, B.Q4_1, B.Q5_0, B.Q5_1, B.Q5_K) for (M, K, n) in SHAPES]
CASES += [(Q4_K, 300, 2304, 6), (Q4_K, 129, 14336, 7), (Q4_K, 1000, 4096, 8)]


@pytest.mark.parametrize("wtype,M,K,n", CASES, ids=[f"{TNAME[c[0]]}-{c[1]}x{c[2]}-n{c[3]}" for c in CASES])
def test_many_columns_parity(O, wtype, M, K, n):
    announce(f"mmvq many columns {TNAME[wtype]} M={M} K={K} n={n}")
    rng = np.random.default_rng(M + K + n + 7 * wtype)
    W = synth.weights(wtype, M, K, rng)
    x = synth.activations(K, n, rng)
    yd = gpu_quantize(x)
    y = O.quantize_q8_1(x)
    assert np.array_equal(host(yd), y)
    out = _nan(n, M)
    B.mmvq(dev(W), wtype, M, K, yd, n, out)
    ref, mag, _ = O.mmvq(W, wtype, M, K, y, n)
    assert_close(host(out), ref, mag, f"many columns {TNAME[wtype]} {M}x{K} n={n}")


@pytest.mark.parametrize("name,n", [("q4_k_4096x14336", 64), ("q6_k_128256x4096", 16), ("q8_0_4096x14336", 32),
                                    ("q4_1_4096x14336", 16), ("q5_0_4096x14336", 9), ("q5_1_4096x14336", 32),
                                    ("q5_k_4096x14336", 16)])
def test_many_columns_workload(O, name, n):
    """The FFN-down and LM-head shapes with many columns, the launches the
    benchmark times; every row and column against the oracle."""
    wl = synth.BY_NAME[name]
    announce(f"mmvq many columns workload {name} n={n}")
    rng = np.random.default_rng(4242 + n)
    W = synth.make(wl, 1)["W"]
    x = synth.activations(wl.K, n, rng)
    yd = gpu_quantize(x)
    y = O.quantize_q8_1(x)
    out = _nan(n, wl.M)
    B.mmvq(dev(W), wl.wtype, wl.M, wl.K, yd, n, out)
    ref, mag = O.mmvq_threaded(W, wl.wtype, wl.M, wl.K, y, n)
    assert_close(host(out), ref, mag, f"many columns workload {name} n={n}")


@pytest.mark.parametrize("wtype", [Q4_K, Q6_K, B.Q5_K])
def test_many_columns_glu_workload(O, wtype):
    """The gate/up form at the FFN-up shape (14336x4096), 16 columns: every
    output against the oracle's gate/up product within the propagated
    tolerance."""
    M, K, n = 14336, 4096, 16
    announce(f"mmvq_glu many columns {TNAME[wtype]} M={M} K={K} n={n}")
    rng = np.random.default_rng(99 + wtype)
    Wu = synth.weights(wtype, M, K, rng)
    Wg = synth.weights(wtype, M, K, rng)
    x = synth.activations(K, n, rng)
    y = O.quantize_q8_1(x)
    out = _nan(n, M)
    B.mmvq_glu(dev(Wg), dev(Wu), wtype, M, K, gpu_quantize(x), n, B.GLU_SWIGLU, out)
    u, mu = O.mmvq_threaded(Wu, wtype, M, K, y, n)
    g, mg = O.mmvq_threaded(Wg, wtype, M, K, y, n)
    ref = O.mmvq_glu(Wg, Wu, wtype, M, K, y, n, B.GLU_SWIGLU)
    tol = glu_tolerance(g, u, mg, mu, ref, B.GLU_SWIGLU)
    got = host(out).astype(np.float64)
    bad = ~(np.abs(got - ref) <= tol)
    assert not bad.any(), f"first bad at {np.argwhere(bad)[0]}"


# Beyond 8 columns the forms the matrix-core kernel does not take (K not a
# multiple of 256) run as groups of 8 columns through the row kernels; the
# fp32 and gate/up forms take the matrix-core kernel when K is a multiple of
# 256.
GROUPS = [(Q4_0, 37, 96, 12), (Q8_0, 300, 1056, 17), (Q6_K, 17, 768, 9), (Q4_K, 129, 4096, 20),
          (B.Q4_1, 37, 1056, 12), (B.Q5_0, 17, 1056, 9), (B.Q5_1, 33, 512, 20), (B.Q5_K, 65, 2048, 16)]


@pytest.mark.parametrize("wtype,M,K,n", GROUPS, ids=[f"{TNAME[c[0]]}-{c[1]}x{c[2]}-n{c[3]}" for c in GROUPS])
def test_column_groups(O, wtype, M, K, n):
    """q8_1 (K not a multiple of 256 for Q4_0 / Q8_0 / Q4_1 / Q5_0), fp32 and
    gate/up forms with more than 8 columns, against the oracle."""
    announce(f"column groups {TNAME[wtype]} M={M} K={K} n={n}")
    rng = np.random.default_rng(M * 3 + K + n)
    Wu = synth.weights(wtype, M, K, rng)
    Wg = synth.weights(wtype, M, K, rng)
    ldx = K + 3
    x = synth.activations(K, n, rng, ldx)
    y = O.quantize_q8_1(x, K)
    yd = gpu_quantize(x, K)
    u, mu, _ = O.mmvq(Wu, wtype, M, K, y, n)
    g, mg, _ = O.mmvq(Wg, wtype, M, K, y, n)
    if K % 256:
        out = _nan(n, M)
        B.mmvq(dev(Wu), wtype, M, K, yd, n, out)
        assert_close(host(out), u, mu, "q8_1 column groups")
    out = _nan(n, M)
    B.mmvq_f32(dev(Wu), wtype, M, K, dev(x), n, ldx, out)
    assert_close(host(out), u, mu, "fp32 column groups")
    out = _nan(n, M)
    B.mmvq_glu(dev(Wg), dev(Wu), wtype, M, K, yd, n, B.GLU_SWIGLU, out)
    ref = O.mmvq_glu(Wg, Wu, wtype, M, K, y, n, B.GLU_SWIGLU)
    tol = glu_tolerance(g, u, mg, mu, ref, B.GLU_SWIGLU)
    got = host(out).astype(np.float64)
    bad = ~(np.abs(got - ref) <= tol)
    assert not bad.any(), f"gate/up column groups: first bad at {np.argwhere(bad)[0]}"


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
    assert L.mmvq(p, B.Q4_0, 1, 256, q, 257, o, s) == B.ERR_SHAPE
    assert L.mmvq(p, B.Q6_K, 1, 96, q, 9, o, s) == B.ERR_SHAPE
    assert L.mmvq(p, 5, 1, 256, q, 9, o, s) == B.ERR_TYPE
    assert L.mmvq(p, Q4_K, 1, 200, q, 9, o, s) == B.ERR_SHAPE
    assert L.mmvq(p + 4, Q4_K, 1, 256, q, 9, o, s) == B.ERR_ALIGN
    assert L.mmvq(p + 4, B.Q8_0, 1, 96, q, 9, o, s) == B.ERR_ALIGN     # column groups check first
    assert L.mmvq_glu(p, p, Q4_K, 1, 256, q, 257, 1, o, s) == B.ERR_SHAPE
    assert L.mmvq_f32(p, Q4_K, 1, 256, o, 257, 256, o, s) == B.ERR_SHAPE
    # the fp32 form on the matrix-core kernel checks its column stride and alignment
    assert L.mmvq_f32(p, Q4_K, 1, 256, o, 9, 255, o, s) == B.ERR_SHAPE
    assert L.mmvq_f32(p, Q4_K, 1, 256, o + 2, 9, 256, o, s) == B.ERR_ALIGN
    assert L.mmvq_f32(p + 4, Q4_K, 1, 256, o, 9, 256, o, s) == B.ERR_ALIGN
    assert L.mmvq_glu_f32(p, p + 4, Q4_K, 1, 256, o, 9, 256, 1, o, s) == B.ERR_ALIGN
    torch.cuda.synchronize()
