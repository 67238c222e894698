"""Shared helpers of the GPU parity tests: device transfer, the oracle
comparison with the stated tolerances, and case announcements (printed and
flushed before each GPU step so a failing run names its case)."""
from __future__ import annotations

import sys

import numpy as np

from quantized_decode_gemv_quantize_amd import binding as B
from quantized_decode_gemv_quantize_amd import synth

TNAME = {B.Q4_0: "q4_0", B.Q8_0: "q8_0", B.Q4_K: "q4_k", B.Q6_K: "q6_k",
         B.Q4_1: "q4_1", B.Q5_0: "q5_0", B.Q5_1: "q5_1", B.Q5_K: "q5_k"}

# |gpu - oracle| <= REL * A + ABS, with A the sum of |block contributions|.
REL, ABS = 1e-5, 1e-6


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_quantize(x: np.ndarray, K: int | None = None):
    """x float32 [n, ldx] -> device q8_1 [n, K/32*36] (uint8)."""
    import torch
    xd = dev(x.astype(np.float32))
    n, ldx = x.shape
    K = ldx if K is None else K
    y = torch.zeros((n, K // 32 * 36), dtype=torch.uint8, device="cuda:0")
    B.mmvq_quantize_q8_1(xd, K, n, ldx, y)
    return y


def gpu_gemv(Wd, wtype, M, K, yd, n):
    import torch
    out = torch.full((n, M), float("nan"), dtype=torch.float32, device="cuda:0")
    B.mmvq(Wd, wtype, M, K, yd, n, out)
    return host(out)


def assert_close(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, what: str) -> None:
    """Finite oracle values: within the tolerance. Non-finite ones (a q8_1
    block sum s that overflowed fp16 to inf): the same inf, or NaN for NaN."""
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    tol = np.where(fin, REL * mag + ABS, 0.0)
    with np.errstate(invalid="ignore"):
        err = np.where(fin, np.abs(got - ref), 0.0)
        bad = np.where(fin, ~(err <= tol), ~((got == ref) | (np.isnan(got) & np.isnan(ref))))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside |d| <= {REL}*A + {ABS}; first at "
            f"{tuple(int(v) for v in i)}: gpu {got[tuple(i)]!r} oracle {ref[tuple(i)]!r} "
            f"A {mag[tuple(i)]!r} (max err/tol {float(np.max(np.where(fin, err / np.where(fin, tol, 1), 0))):.3g})")


def glu_tolerance(g, u, mg, mu, out, op):
    """Bound for act(g)*u given per-dot bounds tg, tu of g and u:
    |d(act(g)*u)| <= |act'(g)|*|u|*tg + |act(g)|*tu + (GPU exp) 1e-6*|out| + ABS,
    with |silu'| <= 1.1 and act' = 1 for the plain product."""
    tg = REL * mg + ABS
    tu = REL * mu + ABS
    if op == B.GLU_SWIGLU:
        act = g / (1.0 + np.exp(-g))
        dact = 1.1
    else:
        act = g
        dact = 1.0
    return dact * np.abs(u) * tg + np.abs(act) * tu + 1e-6 * np.abs(out) + ABS


def special_x(K: int, n: int, seed: int, ldx: int | None = None) -> np.ndarray:
    """N(0,1) activations with some blocks replaced by edge cases: all zero,
    exact .5 ties at d = 1, fp32 subnormals, large values (s overflows fp16),
    a single nonzero element, constant blocks, values within a few ulps of
    the code boundaries."""
    rng = np.random.default_rng(seed)
    x = synth.activations(K, n, rng, ldx)
    nb = K // 32
    for j in range(n):
        for b in range(nb):
            kind = (b + 3 * j) % 9
            blk = x[j, 32 * b:32 * b + 32]
            if kind == 1:
                blk[:] = 0
            elif kind == 2:
                blk[:] = (rng.integers(-100, 100, 32) + 0.5).astype(np.float32)
                blk[0] = 127.0
            elif kind == 3:
                blk[:] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-40)
            elif kind == 4:
                blk[:] = rng.standard_normal(32).astype(np.float32) * np.float32(3e4)
            elif kind == 5:
                blk[:] = 0
                blk[int(rng.integers(0, 32))] = -7.25
            elif kind == 6:
                blk[:] = 2.0
            elif kind == 7:
                # values within a few ulps of (k + 1/2) * d, the code
                # boundaries, for a scale d that is not a power of two
                amax = np.float32(88.9) * np.float32(1 + j)
                d = np.float32(amax / np.float32(127))
                k = rng.integers(0, 127, 32).astype(np.float32)
                t = ((k + np.float32(0.5)) * d).astype(np.float32)
                steps = rng.integers(-4, 5, 32)
                t = np.array([np.float32(v) + np.float32(s) * np.spacing(np.float32(v))
                              for v, s in zip(t, steps)], dtype=np.float32)
                t = np.minimum(t, amax) * np.where(rng.random(32) < 0.5, -1, 1).astype(np.float32)
                t[0] = amax
                blk[:] = t
    return x


def epilogue_tolerance(g, u, mg, mu, epi: dict, e_idx=None):
    """Bound on |gpu - oracle| for the full epilogue out = GLU(g*sg + bg,
    u*su + bu) (or u*su + bu without a gate: g None), from the per-dot bounds
    of the raw up and gate products (REL*mag + ABS), the fp32 rounding of the
    scale and bias steps, and the derivatives of each GLU: |d/dg| and |d/du|
    bounded by 1.1*|u'| and |silu| (SWIGLU), 1.13*|u'| and |gelu| (GEGLU,
    tanh form, |gelu'| <= 1.13), (1 + alpha*|g'|/4)*|u'+1| and
    |g' sigmoid(alpha g')| (OAI, alpha 1.702 and limit 7 of its published
    form), as SWIGLU on the clamped values (CLAMP, the caller's limit); the
    device exp/tanh add 1e-6*(|out| + |g*u|). e_idx: per-row expert index
    for the scales and bias rows (id form), else expert 0."""
    M = u.shape[-1]
    rows = np.arange(M)
    e = np.zeros(u.shape, dtype=np.int64) if e_idx is None else e_idx

    def apply(v, mag, scale, bias):
        tol = REL * mag + ABS
        sc = np.ones_like(v) if scale is None else np.asarray(scale, dtype=np.float64)[e]
        b = np.zeros_like(v) if bias is None else np.asarray(bias, dtype=np.float64).reshape(-1)[e * M + rows]
        w = v * sc + b
        return w, np.abs(sc) * tol + 2.0 ** -23 * (np.abs(v * sc) + np.abs(b)) * 2

    uu, tu = apply(u, mu, epi.get("up_scale"), epi.get("up_bias"))
    if g is None:
        return uu, tu
    gg, tg = apply(g, mg, epi.get("gate_scale"), epi.get("gate_bias"))
    op, L = epi.get("glu_op", 0), epi.get("limit", 0.0)
    if op == 3:
        L, a = 7.0, 1.702
    gc = np.minimum(gg, L)
    uc = np.clip(uu, -L, L)
    silu = lambda z: z / (1.0 + np.exp(-z))  # noqa: E731
    if op == 0:
        out, dg, du = gg * uu, np.abs(uu), np.abs(gg)
    elif op == 1:
        out, dg, du = silu(gg) * uu, 1.1 * np.abs(uu), np.abs(silu(gg))
    elif op == 2:
        gel = 0.5 * gg * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (gg + 0.044715 * gg ** 3)))
        out, dg, du = gel * uu, 1.13 * np.abs(uu), np.abs(gel)
    elif op == 3:
        h = gc / (1.0 + np.exp(-a * gc))
        out, dg, du = h * (uc + 1.0), (1.0 + a * np.abs(gc) / 4.0) * np.abs(uc + 1.0), np.abs(h)
    else:
        out, dg, du = silu(gc) * uc, 1.1 * np.abs(uc), np.abs(silu(gc))
    tol = dg * tg + du * tu + 1e-6 * (np.abs(out) + np.abs(gg * uu)) + ABS
    return out, tol
