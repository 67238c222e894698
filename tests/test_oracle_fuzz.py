"""Property-based fuzzing of the oracle (hypothesis): on drawn shapes, weight
blocks and activations, the integer-dot formulation equals the fp64
dequantize-then-dot brute force written in the test (the pin's dequantizers),
and q8_1 quantization keeps its invariants (|q| <= 127, the largest |x| of a
block maps to |q| = 127, zero blocks give zero d, s and codes)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from oracle_pins import BLOCK, DEQ, deq_y
from quantized_decode_gemv_quantize_amd import synth

Q4_0, Q8_0, Q4_K, Q6_K = oracle.Q4_0, oracle.Q8_0, oracle.Q4_K, oracle.Q6_K
Q4_1, Q5_0, Q5_1, Q5_K = oracle.Q4_1, oracle.Q5_0, oracle.Q5_1, oracle.Q5_K
LEGACY = (Q4_0, Q4_1, Q5_0, Q5_1)      # offset term from the q8_1 block's fp16 s

SETTINGS = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(scope="module")
def O():
    return oracle.default()


# activations: finite fp32 values spanning magnitudes, zeros and exact halves
_elem = st.one_of(st.floats(-1e3, 1e3, width=32, allow_nan=False, allow_infinity=False),
                  st.sampled_from([0.0, 0.5, -0.5, 127.0, -1.5, 1e-30, 2.5]))


@st.composite
def gemv_case(draw):
    wtype = draw(st.sampled_from([Q4_0, Q8_0, Q4_K, Q6_K, Q4_1, Q5_0, Q5_1, Q5_K]))
    qk, _ = BLOCK[wtype]
    nblk = draw(st.integers(1, 3 if qk == 256 else 6))
    K = nblk * qk
    M = draw(st.integers(1, 3))
    n = draw(st.integers(1, 2))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    x = draw(hnp.arrays(np.float32, (n, K), elements=_elem))
    scale = draw(st.sampled_from([1.0, 1e-3, 64.0]))     # scales the drawn fp16 weight scales
    return wtype, M, K, n, seed, x, scale


def _rescale(W, wtype, scale):
    """Multiply every fp16 block scale of W by `scale` (a power of two or
    1e-3, values stay finite)."""
    qk, bb = BLOCK[wtype]
    W = W.copy().reshape(-1, bb)
    fields = {Q4_0: [(0, 2)], Q8_0: [(0, 2)], Q4_K: [(0, 2), (2, 4)], Q6_K: [(208, 210)],
              Q4_1: [(0, 2), (2, 4)], Q5_0: [(0, 2)], Q5_1: [(0, 2), (2, 4)], Q5_K: [(0, 2), (2, 4)]}[wtype]
    for a, b in fields:
        v = W[:, a:b].copy().view(np.float16).astype(np.float64) * scale
        W[:, a:b] = v.astype(np.float16).view(np.uint8)
    return W.reshape(-1)


@SETTINGS
@given(gemv_case())
def test_oracle_equals_dequantized_dot(O, case):
    wtype, M, K, n, seed, x, scale = case
    W = _rescale(synth.weights(wtype, M, K, np.random.default_rng(seed)), wtype, scale)
    y = O.quantize_q8_1(x)
    out, mag, _ = O.mmvq(W, wtype, M, K, y, n)
    row_bytes = K // BLOCK[wtype][0] * BLOCK[wtype][1]
    for j in range(n):
        yd = deq_y(y[j], K)
        for r in range(M):
            w = DEQ[wtype](W[r * row_bytes:(r + 1) * row_bytes], K)
            ref = float(np.dot(w, yd))
            if not np.isfinite(out[j, r]):
                # a q8_1 s that overflowed fp16 (only the old-style formats read s)
                assert wtype in LEGACY
                continue
            if wtype in LEGACY:
                bb = BLOCK[wtype][1]
                yb = y[j].reshape(-1, 36)
                d8 = yb[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1)
                s8 = yb[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)
                sq = yb[:, 4:36].view(np.int8).astype(np.int64).sum(axis=1)
                wb = W[r * row_bytes:(r + 1) * row_bytes].reshape(-1, bb)
                dw = np.abs(wb[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1))
                off = {Q4_0: 8 * dw, Q5_0: 16 * dw}.get(
                    wtype, np.abs(wb[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)))
                tol = float(np.sum(off * np.abs(s8 - d8 * sq))) * (1 + 1e-9) + 1e-12 * mag[j, r] + 1e-300
            else:
                tol = 1e-12 * mag[j, r] + 1e-300
            assert abs(out[j, r] - ref) <= tol, (wtype, K, j, r, out[j, r], ref)


@SETTINGS
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 2), st.integers(1, 4).map(lambda b: 32 * b)),
                  elements=_elem))
def test_q8_1_invariants(O, x):
    y = O.quantize_q8_1(x).reshape(-1, 36)
    xb = x.reshape(-1, 32).astype(np.float64)
    d_h = y[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1)
    s_h = y[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)
    q = y[:, 4:36].view(np.int8).astype(np.int64)
    assert np.all(np.abs(q) <= 127)
    amax = np.abs(xb).max(axis=1)
    for b in range(xb.shape[0]):
        if amax[b] == 0:
            assert d_h[b] == 0 and s_h[b] == 0 and not q[b].any()
        elif amax[b] / 127.0 >= 2.0 ** -126:          # d is a normal fp32
            assert abs(q[b, int(np.argmax(np.abs(xb[b])))]) == 127
            assert np.all(np.sign(q[b]) * np.sign(xb[b]) >= 0)
