"""GPU parity of the fused fp32-activation entry points (mmvq_f32,
mmvq_glu_f32, mmvq_id_f32, mmvq_id_glu_f32).

Each must equal, bit for bit, the q8_1 quantizer followed by the matching
q8_1 entry point on the same inputs (the row kernels quantize in their
prologue, the many-column kernel in its staging, both with the quantizer's
arithmetic; where only one of the two forms runs the many-column kernel,
both against the oracle instead), and be within the oracle tolerance of the
oracle's quantize-then-multiply. Activations include the quantizer's edge cases
(zero, tie, subnormal, large and constant blocks) and column strides that
are not multiples of 4 floats; column counts span the row kernels (1..8),
the many-column kernel (from the library's crossover up to 256) and the
column groups of the forms it does not take.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TNAME, announce, assert_close, dev, glu_tolerance, gpu_quantize, host, special_x
from quantized_decode_gemv_quantize_amd import binding as B
from quantized_decode_gemv_quantize_amd import synth

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = B.Q4_0, B.Q8_0, B.Q4_K, B.Q6_K
Q4_1, Q5_0, Q5_1, Q5_K = B.Q4_1, B.Q5_0, B.Q5_1, B.Q5_K


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _empty(rows, M):
    import torch
    return torch.full((rows, M), float("nan"), dtype=torch.float32, device="cuda:0")


def _mmq_route(wtype, K, n, gated=False):
    """Where exactly one of the q8_1 and fp32 forms runs the many-column
    kernel (K a multiple of 256, each form from its own crossover): there
    the two sum in different orders and agree within the tolerance, not bit
    for bit."""
    if K % 256:
        return False
    return (n >= B.mmvq_many_columns_min(wtype, gated)) != (n >= B.mmvq_many_columns_min(wtype, gated, fp32=True))


def _same(a, b, what):
    """Bit-for-bit equality of two fp32 device tensors (NaN and inf included)."""
    import torch
    torch.cuda.synchronize()
    ai, bi = a.view(torch.int32), b.view(torch.int32)
    if not torch.equal(ai, bi):
        diff = ai != bi
        i = tuple(int(v) for v in diff.nonzero()[0])
        raise AssertionError(f"{what}: fused {a[i].item()!r} != two-step {b[i].item()!r} at {i} "
                             f"({int(diff.sum())} differ)")


FUSED_CASES = [(Q4_0, 37, 96, 1, 0), (Q4_0, 300, 1024, 3, 5), (Q4_0, 129, 16384, 8, 1),
               (Q4_K, 1, 256, 1, 0), (Q4_K, 37, 512, 2, 3), (Q4_K, 1000, 4096, 5, 0),
               (Q4_K, 129, 14336, 8, 7), (Q4_K, 65, 16384, 1, 1), (Q4_K, 33, 32768, 1, 2),
               (Q4_K, 20, 32768, 8, 3),
               (Q6_K, 1, 256, 1, 0), (Q6_K, 37, 768, 3, 2), (Q6_K, 300, 4096, 8, 0),
               (Q6_K, 129, 32768, 2, 1), (Q8_0, 37, 96, 1, 0), (Q8_0, 300, 1024, 3, 5),
               (Q8_0, 129, 16384, 8, 1),
               # enough rows that teams take them in 2 or 4 passes (ragged last team)
               (Q4_K, 12301, 4096, 2, 1), (Q4_K, 12301, 4096, 5, 0), (Q4_0, 12301, 4096, 3, 0),
               (Q8_0, 12301, 4096, 8, 2), (Q6_K, 12301, 4096, 4, 1),
               # rows walked in chunks (ragged last chunk for 16416, 33024, 40000)
               (Q4_K, 37, 65536, 1, 0), (Q4_K, 9, 33024, 8, 3), (Q4_0, 37, 32768, 2, 1),
               (Q4_0, 5, 16416, 5, 0), (Q8_0, 17, 40000, 3, 2), (Q6_K, 17, 65792, 1, 1),
               (Q6_K, 3, 33024, 8, 0),
               # formats the pages name without layouts
               (Q4_1, 37, 96, 1, 0), (Q4_1, 300, 1024, 3, 5), (Q5_0, 37, 1056, 2, 1), (Q5_0, 129, 4096, 8, 0),
               (Q5_1, 300, 1024, 5, 3), (Q5_K, 1000, 4096, 1, 0), (Q5_K, 129, 14336, 8, 7),
               (Q5_K, 12301, 4096, 2, 1),
               # pipelined rows (few waves per CU, 8 or 16 rows per team)
               (Q4_1, 4096, 4096, 1, 0), (Q5_1, 4096, 4096, 1, 2), (Q5_K, 4096, 4096, 1, 1),
               (Q5_K, 2048, 14336, 1, 0),
               # the one-column single-team-per-workgroup kernel, ragged last team
               (Q4_K, 4099, 14336, 1, 3), (Q4_1, 4100, 8192, 1, 0), (Q5_1, 2055, 16384, 1, 1),
               # many columns: the matrix-core kernel quantizing its staged blocks
               # (ragged row and column tiles, up to the 256-column maximum), and
               # column groups through the row kernels where K is not a multiple of 256
               (Q4_K, 300, 4096, 16, 3), (Q4_K, 129, 14336, 33, 1), (Q4_K, 37, 512, 256, 2),
               (Q4_K, 1000, 2048, 6, 0), (Q6_K, 37, 768, 9, 2), (Q6_K, 300, 2304, 40, 0),
               (Q4_0, 300, 1024, 40, 5), (Q8_0, 65, 2048, 17, 0), (Q4_1, 33, 1280, 24, 1),
               (Q5_0, 70, 768, 9, 0), (Q5_1, 17, 1280, 64, 2), (Q5_K, 129, 4096, 16, 1),
               (Q5_K, 9000, 512, 5, 3), (Q4_0, 37, 96, 20, 1), (Q8_0, 33, 1056, 12, 2),
               (Q6_K, 300, 2048, 6, 1), (Q6_K, 129, 4096, 8, 0), (Q5_K, 300, 2048, 8, 2)]


@pytest.mark.parametrize("wtype,M,K,n,pad", FUSED_CASES,
                         ids=[f"{TNAME[c[0]]}-{c[1]}x{c[2]}-n{c[3]}-pad{c[4]}" for c in FUSED_CASES])
def test_mmvq_f32(O, wtype, M, K, n, pad):
    announce(f"mmvq_f32 {TNAME[wtype]} M={M} K={K} n={n} ldx=K+{pad}")
    rng = np.random.default_rng(31 * M + K + n)
    W = synth.weights(wtype, M, K, rng)
    x = special_x(K, n, seed=M + n, ldx=K + pad)
    Wd, xd = dev(W), dev(x)
    fused, two = _empty(n, M), _empty(n, M)
    B.mmvq_f32(Wd, wtype, M, K, xd, n, K + pad, fused)
    yd = gpu_quantize(x, K)
    B.mmvq(Wd, wtype, M, K, yd, n, two)
    y = O.quantize_q8_1(x, K)
    ref, mag, _ = O.mmvq(W, wtype, M, K, y, n)
    if _mmq_route(wtype, K, n):
        assert_close(host(two), ref, mag, f"mmvq {TNAME[wtype]} {M}x{K} n={n}")
    else:
        _same(fused, two, f"mmvq_f32 {TNAME[wtype]} {M}x{K} n={n}")
    assert_close(host(fused), ref, mag, f"mmvq_f32 {TNAME[wtype]} {M}x{K} n={n}")


GLU_F32 = [(Q4_K, 300, 4096, 1, B.GLU_SWIGLU), (Q4_K, 37, 512, 4, B.GLU_PLAIN),
           (Q4_0, 300, 1024, 2, B.GLU_SWIGLU), (Q6_K, 37, 768, 3, B.GLU_SWIGLU),
           (Q4_K, 129, 14336, 8, B.GLU_SWIGLU), (Q4_K, 17, 65536, 2, B.GLU_SWIGLU),
           (Q8_0, 9, 16416, 8, B.GLU_PLAIN),
           # many columns (matrix-core kernel, and column groups for K % 256 != 0)
           (Q4_K, 300, 4096, 16, B.GLU_SWIGLU), (Q4_K, 129, 2048, 7, B.GLU_GEGLU),
           (Q5_K, 129, 2048, 9, B.GLU_GEGLU), (Q6_K, 37, 768, 33, B.GLU_SWIGLU),
           (Q8_0, 65, 1024, 12, B.GLU_PLAIN), (Q4_0, 17, 1056, 11, B.GLU_SWIGLU),
           # the gate/up fp32 form on the many-column kernel from 4 or 5 columns
           (Q4_0, 300, 1024, 4, B.GLU_SWIGLU), (B.Q5_0, 129, 2048, 6, B.GLU_GEGLU),
           (Q5_K, 65, 1024, 4, B.GLU_SWIGLU), (Q4_K, 300, 2048, 5, B.GLU_SWIGLU),
           (Q6_K, 37, 768, 5, B.GLU_PLAIN), (Q8_0, 129, 1024, 8, B.GLU_SWIGLU),
           (B.Q4_1, 65, 512, 7, B.GLU_SWIGLU), (B.Q5_1, 33, 1280, 6, B.GLU_GEGLU)]


@pytest.mark.parametrize("wtype,M,K,n,op", GLU_F32,
                         ids=[f"{TNAME[c[0]]}-{c[1]}x{c[2]}-n{c[3]}-op{c[4]}" for c in GLU_F32])
def test_mmvq_glu_f32(O, wtype, M, K, n, op):
    announce(f"mmvq_glu_f32 {TNAME[wtype]} M={M} K={K} n={n} op={op}")
    rng = np.random.default_rng(M + K + 17 * n + op)
    Wg, Wu = synth.weights(wtype, M, K, rng), synth.weights(wtype, M, K, rng)
    ldx = K + 1
    x = synth.activations(K, n, rng, ldx)
    Wgd, Wud, xd = dev(Wg), dev(Wu), dev(x)
    fused, two = _empty(n, M), _empty(n, M)
    B.mmvq_glu_f32(Wgd, Wud, wtype, M, K, xd, n, ldx, op, fused)
    B.mmvq_glu(Wgd, Wud, wtype, M, K, gpu_quantize(x, K), n, op, two)
    routed = _mmq_route(wtype, K, n, gated=True)
    if not routed:
        _same(fused, two, f"mmvq_glu_f32 {TNAME[wtype]} {M}x{K} n={n}")
    y = O.quantize_q8_1(x, K)
    g, mg, _ = O.mmvq(Wg, wtype, M, K, y, n)
    u, mu, _ = O.mmvq(Wu, wtype, M, K, y, n)
    ref = O.mmvq_glu(Wg, Wu, wtype, M, K, y, n, op)
    tol = glu_tolerance(g, u, mg, mu, ref, op)
    for out in ([fused, two] if routed else [fused]):
        got = host(out).astype(np.float64)
        bad = ~(np.abs(got - ref) <= tol)
        assert not bad.any(), f"first bad at {np.argwhere(bad)[0]}"


ID_F32 = [("q4_k-E4-T3-k2", Q4_K, 4, 200, 512, [[2, 0], [1, 2], [2, 3]]),
          ("q4_k-E8-T8-k2", Q4_K, 8, 300, 2048, "random"),
          # fewer rows than the fp32 gate/up kernel's 32-row expert blocks
          ("q4_k-E3-T4-k2-M20", Q4_K, 3, 20, 512, [[2, 0], [1, 2], [0, 1], [2, 1]]),
          ("q4_0-E5-T4-k2", Q4_0, 5, 77, 1024, [[4, 0], [0, 4], [2, 2], [1, 3]]),
          ("q6_k-E4-T2-k2", Q6_K, 4, 50, 768, [[3, 1], [1, 0]]),
          # rows walked in chunks
          ("q4_k-E2-T3-k2-K65536", Q4_K, 2, 17, 65536, [[1, 0], [0, 1], [1, 1]]),
          ("q8_0-E3-T8-k2-K16416", Q8_0, 3, 9, 16416, "random")]


@pytest.mark.parametrize("fused_glu", [False, True])
@pytest.mark.parametrize("name,wtype,E,M,K,ids", ID_F32, ids=[c[0] for c in ID_F32])
def test_mmvq_id_f32(O, name, wtype, E, M, K, ids, fused_glu):
    announce(f"mmvq_id{'_glu' if fused_glu else ''}_f32 {name}")
    if isinstance(ids, str):
        ids = synth.expert_ids(8, 2, E, np.random.default_rng(5))
    ids = np.asarray(ids, dtype=np.int32)
    T, top_k = ids.shape
    rng = np.random.default_rng(len(name) + 100)
    Wu = np.stack([synth.weights(wtype, M, K, rng) for _ in range(E)])
    Wg = np.stack([synth.weights(wtype, M, K, rng) for _ in range(E)])
    ldx = K + 2
    x = synth.activations(K, T, rng, ldx)
    stride = (Wu[0].size + 15) // 16 * 16
    pad = lambda A: np.concatenate(  # noqa: E731
        [np.pad(A[e].reshape(-1), (0, stride - A[e].size)) for e in range(E)])
    Wud, Wgd, xd, idsd = dev(pad(Wu)), dev(pad(Wg)), dev(x), dev(ids)
    fused, two = _empty(T * top_k, M), _empty(T * top_k, M)
    yd = gpu_quantize(x, K)
    if fused_glu:
        B.mmvq_id_glu_f32(Wgd, Wud, stride, E, wtype, M, K, xd, T, ldx, idsd, top_k, B.GLU_SWIGLU, fused)
        B.mmvq_id_glu(Wgd, Wud, stride, E, wtype, M, K, yd, T, idsd, top_k, B.GLU_SWIGLU, two)
    else:
        B.mmvq_id_f32(Wud, stride, E, wtype, M, K, xd, T, ldx, idsd, top_k, fused)
        B.mmvq_id(Wud, stride, E, wtype, M, K, yd, T, idsd, top_k, two)
    _same(fused, two, f"id f32 {name}")
    _id_against_oracle(O, host(fused), Wu, Wg if fused_glu else None, wtype, M, K, x, ids, f"id f32 {name}")


def _id_against_oracle(O, got, Wu, Wg, wtype, M, K, x, ids, what):
    """Every (token, slot) row of an expert-indexed result against the oracle:
    the up product alone (Wg None) or SWIGLU of the gate and up products."""
    y = O.quantize_q8_1(x, K)
    T, top_k = ids.shape
    got = np.asarray(got, dtype=np.float64)
    for t in range(T):
        for k in range(top_k):
            e, s = int(ids[t, k]), t * top_k + k
            u, mu = O.mmvq_threaded(Wu[e], wtype, M, K, y[t:t + 1], 1)
            if Wg is None:
                assert_close(got[s:s + 1], u, mu, f"{what} token {t} slot {k}")
                continue
            g, mg = O.mmvq_threaded(Wg[e], wtype, M, K, y[t:t + 1], 1)
            ref = O.glu_array(B.GLU_SWIGLU, g, u)
            tol = glu_tolerance(g, u, mg, mu, ref, B.GLU_SWIGLU)
            bad = ~(np.abs(got[s:s + 1] - ref) <= tol)
            assert not bad.any(), f"{what} token {t} slot {k} expert {e}: first {np.argwhere(bad)[0]}"


def test_mmvq_id_glu_f32_moe_workload(O):
    """The MoE workload (8 experts, 8 tokens, top-2, Q4_K 14336x4096 gate
    and up) through the fused fp32 form, in the launch configuration the
    benchmark times: every output bit-identical to quantize + mmvq_id_glu,
    and every row of every slot against the oracle."""
    wl = synth.BY_NAME["moe_q4_k_8x14336x4096"]
    announce("mmvq_id_glu_f32 moe workload")
    d = synth.make(wl, 8)
    E, M, K, top_k = wl.n_experts, wl.M, wl.K, wl.top_k
    ids, x = d["ids"].astype(np.int32), d["x"]
    T = ids.shape[0]
    stride = (d["W_up"][0].size + 15) // 16 * 16
    pad = lambda A: np.concatenate(  # noqa: E731
        [np.pad(A[e].reshape(-1), (0, stride - A[e].size)) for e in range(E)])
    Wud, Wgd, xd, idsd = dev(pad(d["W_up"])), dev(pad(d["W_gate"])), dev(x), dev(ids)
    fused, two = _empty(T * top_k, M), _empty(T * top_k, M)
    B.mmvq_id_glu_f32(Wgd, Wud, stride, E, wl.wtype, M, K, xd, T, x.shape[1], idsd, top_k, B.GLU_SWIGLU, fused)
    B.mmvq_id_glu(Wgd, Wud, stride, E, wl.wtype, M, K, gpu_quantize(x, K), T, idsd, top_k, B.GLU_SWIGLU, two)
    _same(fused, two, "id_glu f32 moe workload")
    _id_against_oracle(O, host(fused), d["W_up"], d["W_gate"], wl.wtype, M, K, x, ids, "id_glu f32 moe workload")


WORKLOADS_F32 = [("q4_k_4096x14336", 1), ("q4_k_4096x14336", 2), ("q4_k_4096x14336", 8),
                 ("q4_k_14336x4096", 4), ("q6_k_128256x4096", 1), ("q6_k_128256x4096", 2),
                 ("q4_0_256x1024", 1), ("q8_0_4096x14336", 1), ("q4_1_4096x14336", 1),
                 ("q5_0_4096x14336", 1), ("q5_1_4096x14336", 1), ("q5_k_4096x14336", 1),
                 ("q4_k_4096x14336", 16), ("q5_k_4096x14336", 16), ("q8_0_4096x14336", 32)]


@pytest.mark.parametrize("name,n", WORKLOADS_F32, ids=[f"{a}-n{b}" for a, b in WORKLOADS_F32])
def test_mmvq_f32_workload(O, name, n):
    """Workload sizes in the launch configuration the benchmark times: all
    rows bit-identical to the two-step path (where only one of the two
    forms runs the many-column kernel: both against the oracle instead),
    and every row against the oracle."""
    wl = synth.BY_NAME[name]
    announce(f"mmvq_f32 workload {name} n={n}")
    d = synth.make(wl, n)
    W, x = d["W"], d["x"]
    M, K = wl.M, wl.K
    Wd, xd = dev(W), dev(x)
    fused, two = _empty(n, M), _empty(n, M)
    B.mmvq_f32(Wd, wl.wtype, M, K, xd, n, x.shape[1], fused)
    B.mmvq(Wd, wl.wtype, M, K, gpu_quantize(x, K), n, two)
    y = O.quantize_q8_1(x, K)
    ref, mag = O.mmvq_threaded(W, wl.wtype, M, K, y, n)
    got = host(fused)
    if _mmq_route(wl.wtype, wl.K, n):
        assert_close(host(two), ref, mag, f"mmvq {name} n={n}")
    else:
        _same(fused, two, f"mmvq_f32 {name} n={n}")
    assert_close(got, ref, mag, f"mmvq_f32 {name} n={n}")


@pytest.mark.parametrize("wtype", [Q4_K, Q5_K])
def test_mmvq_glu_f32_many_columns_workload(O, wtype):
    """The gate/up form at the FFN-up shape (14336x4096) with 16 fp32
    columns, the launch the benchmark times: bit-identical to the quantizer
    followed by the q8_1 gate/up call, and every output against the
    oracle's gate/up product within the propagated tolerance."""
    M, K, n = 14336, 4096, 16
    announce(f"mmvq_glu_f32 many columns workload {TNAME[wtype]} M={M} K={K} n={n}")
    rng = np.random.default_rng(515 + wtype)
    Wu, Wg = synth.weights(wtype, M, K, rng), synth.weights(wtype, M, K, rng)
    x = synth.activations(K, n, rng)
    Wgd, Wud, xd = dev(Wg), dev(Wu), dev(x)
    fused, two = _empty(n, M), _empty(n, M)
    B.mmvq_glu_f32(Wgd, Wud, wtype, M, K, xd, n, K, B.GLU_SWIGLU, fused)
    B.mmvq_glu(Wgd, Wud, wtype, M, K, gpu_quantize(x, K), n, B.GLU_SWIGLU, two)
    _same(fused, two, f"mmvq_glu_f32 workload {TNAME[wtype]}")
    y = O.quantize_q8_1(x, K)
    u, mu = O.mmvq_threaded(Wu, wtype, M, K, y, n)
    g, mg = O.mmvq_threaded(Wg, wtype, M, K, y, n)
    ref = O.mmvq_glu(Wg, Wu, wtype, M, K, y, n, B.GLU_SWIGLU)
    tol = glu_tolerance(g, u, mg, mu, ref, B.GLU_SWIGLU)
    got = host(fused).astype(np.float64)
    bad = ~(np.abs(got - ref) <= tol)
    assert not bad.any(), f"first bad at {np.argwhere(bad)[0]}"


# (n, gated): the row kernel, the many-column kernel on fp32 columns, and
# its gate/up form (both forms on the many-column kernel at these n)
GRAPH_CASES = [(2, False), (16, False), (8, True)]


@pytest.mark.parametrize("n,gated", GRAPH_CASES, ids=[f"n{c[0]}-{'glu' if c[1] else 'plain'}" for c in GRAPH_CASES])
def test_f32_graph_replay(n, gated):
    """One fused launch captured in a HIP graph on a side stream, replayed
    with new activations copied in between (eager work and synchronization
    between replays): every replay equals the eager two-step result."""
    import torch
    announce(f"mmvq_f32 graph replay n={n} gated={gated}")
    rng = np.random.default_rng(78 + n)
    M, K = 1000, 4096
    W = dev(synth.weights(Q4_K, M, K, rng))
    Wg = dev(synth.weights(Q4_K, M, K, rng))
    xs = [dev(synth.activations(K, n, rng)) for _ in range(3)]
    eager = []
    for xv in xs:
        o = _empty(n, M)
        if gated:
            B.mmvq_glu(Wg, W, Q4_K, M, K, B.quantize(xv), n, B.GLU_SWIGLU, o)
        else:
            B.mmvq(W, Q4_K, M, K, B.quantize(xv), n, o)
        eager.append(o)
    torch.cuda.synchronize()
    x_in = xs[0].clone()
    out = _empty(n, M)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        if gated:
            B.mmvq_glu_f32(Wg, W, Q4_K, M, K, x_in, n, K, B.GLU_SWIGLU, out, side)
        else:
            B.mmvq_f32(W, Q4_K, M, K, x_in, n, K, out, side)
    for rep in range(6):
        x_in.copy_(xs[rep % 3])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(out, eager[rep % 3], f"replay {rep}")
        _ = W[:1024].float().sum()
    torch.cuda.synchronize()


def test_f32_errors_on_device():
    import torch
    announce("f32 abi errors")
    W = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0")
    x = torch.zeros(1 << 14, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(1 << 14, dtype=torch.float32, device="cuda:0")
    L = B.lib()
    s = torch.cuda.current_stream().cuda_stream
    p, q, o = W.data_ptr(), x.data_ptr(), out.data_ptr()
    assert L.mmvq_f32(p, Q4_K, 1, 256, q, 1, 255, o, s) == B.ERR_SHAPE
    assert L.mmvq_f32(p, Q4_K, 1, 256, q + 2, 1, 256, o, s) == B.ERR_ALIGN
    assert L.mmvq_f32(p, Q4_K, 1, 256, q, 257, 256, o, s) == B.ERR_SHAPE
    assert L.mmvq_f32(p + 8, Q4_K, 1, 256, q, 1, 256, o, s) == B.ERR_ALIGN
    # x needs only 4-byte alignment: a valid call (zero weights give 0)
    out.fill_(float("nan"))
    assert L.mmvq_f32(p, Q4_K, 1, 256, q + 4, 1, 256, o, s) == 0
    torch.cuda.synchronize()
    assert out[0].item() == 0.0
