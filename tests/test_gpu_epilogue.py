"""GPU parity of the full fused epilogue (mmvq_ex, mmvq_id_ex): per-matrix
or per-expert scales, bias rows, every GLU op, the MoE shared expert, with
q8_1 or fp32 activations, at one to 40 columns (the many-column kernel's
gate/up form beyond 8), against the oracle (orc_mmvq_ex, orc_mmvq_id_ex)
within the propagated tolerance; the reduced forms (no epilogue; GLU only)
equal mmvq / mmvq_glu bit for bit."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TNAME, announce, dev, epilogue_tolerance, gpu_quantize, host
from quantized_decode_gemv_quantize_amd import binding as B
from quantized_decode_gemv_quantize_amd import synth

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = B.Q4_0, B.Q8_0, B.Q4_K, B.Q6_K
OPS = [B.GLU_PLAIN, B.GLU_SWIGLU, B.GLU_GEGLU, B.GLU_SWIGLU_OAI, B.GLU_SWIGLU_CLAMP]


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


def _check(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r} tol {tol[i]!r}")


CASES = [(t, M, K, n, op, gate, f32)
         for (t, M, K) in [(Q4_K, 300, 2048), (Q4_0, 77, 1024), (Q6_K, 65, 768), (Q8_0, 45, 512)]
         for n in (1, 3)
         for op in OPS
         for gate in (True,)
         for f32 in (False, True)]
CASES += [(t, 129, 4096, n, 0, False, f32) for t in (Q4_K, Q6_K) for n in (1, 8) for f32 in (False, True)]
# more than 8 columns: the gate/up form of the many-column kernel (q8_1),
# column groups through the row kernels (fp32)
CASES += [(t, M, K, n, op, True, False)
          for (t, M, K) in [(Q4_K, 300, 2048), (Q4_0, 77, 1024), (Q6_K, 65, 768), (Q8_0, 45, 512),
                            (B.Q4_1, 33, 512), (B.Q5_0, 40, 768), (B.Q5_1, 17, 1024), (B.Q5_K, 100, 1536)]
          for n in (9, 40)
          for op in OPS]
CASES += [(Q4_K, 300, 2048, 17, B.GLU_SWIGLU, True, True), (Q6_K, 65, 768, 12, B.GLU_GEGLU, True, True)]


@pytest.mark.parametrize("wtype,M,K,n,op,gate,f32", CASES,
                         ids=[f"{TNAME[c[0]]}-{c[1]}x{c[2]}-n{c[3]}-op{c[4]}-{'gate' if c[5] else 'nogate'}"
                              f"-{'f32' if c[6] else 'q8'}" for c in CASES])
def test_mmvq_ex(O, wtype, M, K, n, op, gate, f32):
    announce(f"mmvq_ex {TNAME[wtype]} M={M} K={K} n={n} op={op} gate={gate} f32={f32}")
    rng = np.random.default_rng(M + K + 7 * n + 31 * op + 2 * f32)
    Wu = synth.weights(wtype, M, K, rng)
    Wg = synth.weights(wtype, M, K, rng) if gate else None
    x = synth.activations(K, n, rng)
    # biases and scales of the order of the products (|dot| ~ 1..10)
    epi = dict(up_bias=rng.standard_normal(M).astype(np.float32),
               up_scale=np.float32([rng.uniform(0.5, 1.5)]), glu_op=op, limit=3.0)
    if gate:
        epi.update(gate_bias=rng.standard_normal(M).astype(np.float32),
                   gate_scale=np.float32([rng.uniform(0.1, 0.4)]))
    tens = {k: dev(v) for k, v in epi.items() if isinstance(v, np.ndarray)}
    e = B.epilogue(up_bias=tens["up_bias"], up_scale=tens["up_scale"], gate_bias=tens.get("gate_bias"),
                   gate_scale=tens.get("gate_scale"), glu_op=op, glu_limit=3.0)
    out = _nan(n, M)
    Wud, Wgd = dev(Wu), (dev(Wg) if gate else None)
    if f32:
        B.mmvq_ex(Wud, Wgd, wtype, M, K, None, dev(x), K, n, e, out)
    else:
        B.mmvq_ex(Wud, Wgd, wtype, M, K, gpu_quantize(x), None, 0, n, e, out)
    got = host(out)
    y = O.quantize_q8_1(x)
    oepi = {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v) for k, v in epi.items()}
    ref = O.mmvq_ex(Wu, Wg, wtype, M, K, y, n, oepi)
    u, mu, _ = O.mmvq(Wu, wtype, M, K, y, n)
    g, mg = (O.mmvq(Wg, wtype, M, K, y, n)[:2]) if gate else (None, None)
    ref2, tol = epilogue_tolerance(g, u, mg, mu, oepi)
    assert np.allclose(ref, ref2, rtol=1e-12, atol=1e-12)     # the test's composition agrees with the oracle
    _check(got, ref, tol, f"mmvq_ex {TNAME[wtype]} op {op}")


@pytest.mark.parametrize("f32", [False, True])
def test_reduced_forms_bit_identical(f32):
    """No epilogue and no gate is mmvq; GLU only is mmvq_glu (same code)."""
    import torch
    announce(f"mmvq_ex reduced forms f32={f32}")
    rng = np.random.default_rng(5)
    M, K, n = 300, 4096, 2
    Wu, Wg = dev(synth.weights(Q4_K, M, K, rng)), dev(synth.weights(Q4_K, M, K, rng))
    x = synth.activations(K, n, rng)
    xd, yd = dev(x), gpu_quantize(x)
    a, b = _nan(n, M), _nan(n, M)
    act = (None, xd, K) if f32 else (yd, None, 0)
    B.mmvq_ex(Wu, None, Q4_K, M, K, *act, n, None, a)
    if f32:
        B.mmvq_f32(Wu, Q4_K, M, K, xd, n, K, b)
    else:
        B.mmvq(Wu, Q4_K, M, K, yd, n, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    B.mmvq_ex(Wu, Wg, Q4_K, M, K, *act, n, B.epilogue(glu_op=B.GLU_SWIGLU), a)
    if f32:
        B.mmvq_glu_f32(Wg, Wu, Q4_K, M, K, xd, n, K, B.GLU_SWIGLU, b)
    else:
        B.mmvq_glu(Wg, Wu, Q4_K, M, K, yd, n, B.GLU_SWIGLU, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


ID_CASES = [("q4_k-E4-T3-k2", Q4_K, 4, 200, 512, [[2, 0], [1, 2], [2, 3]], B.GLU_SWIGLU),
            ("q4_k-E8-T8-k2-oai", Q4_K, 8, 300, 2048, "random", B.GLU_SWIGLU_OAI),
            ("q4_0-E5-T4-k2-geglu", Q4_0, 5, 77, 1024, [[4, 0], [0, 4], [2, 2], [1, 3]], B.GLU_GEGLU),
            ("q6_k-E4-T2-k2-clamp", Q6_K, 4, 50, 768, [[3, 1], [1, 0]], B.GLU_SWIGLU_CLAMP)]


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("name,wtype,E,M,K,ids,op", ID_CASES, ids=[c[0] for c in ID_CASES])
def test_mmvq_id_ex_shared_expert(O, name, wtype, E, M, K, ids, op, f32):
    import torch
    announce(f"mmvq_id_ex {name} f32={f32}")
    if isinstance(ids, str):
        ids = synth.expert_ids(8, 2, E, np.random.default_rng(5))
    ids = np.asarray(ids, dtype=np.int32)
    T, top_k = ids.shape
    rng = np.random.default_rng(len(name) + 11 * f32)
    Wu = np.stack([synth.weights(wtype, M, K, rng) for _ in range(E)])
    Wg = np.stack([synth.weights(wtype, M, K, rng) for _ in range(E)])
    Su, Sg = synth.weights(wtype, M, K, rng), synth.weights(wtype, M, K, rng)
    x = synth.activations(K, T, rng)
    stride = (Wu[0].size + 15) // 16 * 16
    pad = lambda A: np.concatenate(  # noqa: E731
        [np.pad(A[e].reshape(-1), (0, stride - A[e].size)) for e in range(E)])
    epi = dict(up_bias=rng.standard_normal(E * M).astype(np.float32),
               gate_bias=rng.standard_normal(E * M).astype(np.float32),
               up_scale=rng.uniform(0.5, 1.5, E).astype(np.float32),
               gate_scale=rng.uniform(0.1, 0.4, E).astype(np.float32), glu_op=op, limit=3.0)
    tens = {k: dev(v) for k, v in epi.items() if isinstance(v, np.ndarray)}
    e = B.epilogue(up_bias=tens["up_bias"], gate_bias=tens["gate_bias"], up_scale=tens["up_scale"],
                   gate_scale=tens["gate_scale"], glu_op=op, glu_limit=3.0)
    out, sh = _nan(T * top_k, M), _nan(T, M)
    act = (None, dev(x), K) if f32 else (gpu_quantize(x), None, 0)
    B.mmvq_id_ex(dev(pad(Wu)), dev(pad(Wg)), stride, E, wtype, M, K, *act, T, dev(ids), top_k, e,
                 dev(Su), dev(Sg), sh, out)
    torch.cuda.synchronize()
    got, got_sh = host(out), host(sh)
    y = O.quantize_q8_1(x)
    oepi = {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v) for k, v in epi.items()}
    for t in range(T):
        for k in range(top_k):
            ex = int(ids[t, k])
            u, mu, _ = O.mmvq(Wu[ex], wtype, M, K, y[t:t + 1], 1)
            g, mg, _ = O.mmvq(Wg[ex], wtype, M, K, y[t:t + 1], 1)
            ref, tol = epilogue_tolerance(g, u, mg, mu, oepi, e_idx=np.full((1, M), ex))
            _check(got[t * top_k + k:t * top_k + k + 1], ref, tol, f"{name} token {t} slot {k}")
        u, mu, _ = O.mmvq(Su, wtype, M, K, y[t:t + 1], 1)
        g, mg, _ = O.mmvq(Sg, wtype, M, K, y[t:t + 1], 1)
        ref, tol = epilogue_tolerance(g, u, mg, mu, dict(glu_op=op, limit=3.0))
        _check(got_sh[t:t + 1], ref, tol, f"{name} shared token {t}")
    # the oracle's own id form agrees with the per-slot composition used above
    o_out, o_sh = O.mmvq_id_ex(pad(Wu), pad(Wg), stride, E, wtype, M, K, y, T, ids, top_k, oepi, Su, Sg)
    assert np.all(np.abs(o_out - got) <= 1e-3 * (1 + np.abs(o_out)))
    assert np.all(np.abs(o_sh - got_sh) <= 1e-3 * (1 + np.abs(o_sh)))
