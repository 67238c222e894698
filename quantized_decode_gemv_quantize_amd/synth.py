"""Seeded synthetic inputs for the quantized mat-vec.

This module is the ONLY code shared by the GPU path's tests/benchmark and the
CPU oracle. It holds no arithmetic of the method: it draws random codes,
scales and activations and places them at their byte offsets inside the
block formats. Quantization, decoding and dot products live only in the
HIP library and (independently) in the oracle.

Block layouts (byte offsets inside one block):

* Q4_0, 18 bytes / 32 weights: fp16 ``d`` at 0, 16 bytes of 4-bit codes at 2.
* Q8_0, 34 bytes / 32 weights: fp16 ``d`` at 0, 32 int8 codes at 2 (drawn
  uniform in -127..127).
* Q4_K, 144 bytes / 256 weights: fp16 ``d`` at 0, fp16 ``dmin`` at 2,
  12 bytes of packed 6-bit scales and mins at 4, 128 bytes of 4-bit codes at 16.
* Q6_K, 210 bytes / 256 weights: 128 bytes of low code bits at 0, 64 bytes of
  high code bits at 128, 16 int8 sub-block scales at 192, fp16 ``d`` at 208.
* Q4_1, 20 bytes / 32 weights: fp16 ``d`` at 0, fp16 ``m`` at 2, 16 bytes of
  4-bit codes at 4.
* Q5_0, 22 bytes / 32 weights: fp16 ``d`` at 0, 4 bytes of fifth code bits at
  2, 16 bytes of 4-bit codes at 6.
* Q5_1, 24 bytes / 32 weights: fp16 ``d`` at 0, fp16 ``m`` at 2, 4 bytes of
  fifth code bits at 4, 16 bytes of 4-bit codes at 8.
* Q5_K, 176 bytes / 256 weights: fp16 ``d`` at 0, fp16 ``dmin`` at 2, 12 bytes
  of packed 6-bit scales and mins at 4, 32 bytes of fifth code bits at 16, 128
  bytes of 4-bit codes at 48.

Every bit pattern of the packed code bytes and of the 12 Q4_K (and Q5_K)
scale bytes is a valid encoding, and uniform random bytes give codes uniform
over their range (4-bit 0..15, 5-bit 0..31, 6-bit 0..63) and 6-bit
scales/mins uniform over 0..63, so those fields are drawn as raw bytes. The
fp16 offsets ``m`` of Q4_1 / Q5_1 are drawn uniform in -8*d_max..0 (a
block's values then straddle zero). The fp16 scales are drawn as fp32 uniforms and
rounded to fp16 by numpy; the Q6_K int8 scales are drawn uniform in -64..63.

Workloads (decode-time layer shapes of a 7B/8B-class model):

=====================  ======  =====  =====  =====  ===========================
name                   type    M      K      n      notes
=====================  ======  =====  =====  =====  ===========================
q4_0_256x1024          Q4_0    256    1024   1      d ~ U[0.001, 0.02]
q4_k_4096x4096         Q4_K    4096   4096   1      attention projection
q4_k_14336x4096        Q4_K    14336  4096   1..8   FFN up/gate
q4_k_4096x14336        Q4_K    4096   14336  1..8   FFN down (headline)
q6_k_128256x4096       Q6_K    128256 4096   1      LM head
moe_q4_k_8x14336x4096  Q4_K    14336  4096   8 tok  8 experts, top-2, gate+up
q8_0_4096x14336        Q8_0    4096   14336  1      FFN down, 8-bit weights
q4_1_4096x14336        Q4_1    4096   14336  1      FFN down, other formats:
q5_0_4096x14336        Q5_0    4096   14336  1      Q4_1, Q5_0, Q5_1, Q5_K
q5_1_4096x14336        Q5_1    4096   14336  1
q5_k_4096x14336        Q5_K    4096   14336  1
=====================  ======  =====  =====  =====  ===========================

Seeds: ``seed = 1000 + workload index``; independent sub-streams are spawned
from it in the order weights, activations, expert ids.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q4_0, Q8_0, Q8_1, Q4_K, Q6_K = 2, 8, 9, 12, 14
Q4_1, Q5_0, Q5_1, Q5_K = 3, 6, 7, 13
BLOCK = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210), Q8_1: (32, 36),
         Q4_1: (32, 20), Q5_0: (32, 22), Q5_1: (32, 24), Q5_K: (256, 176)}
TYPE_NAME = {Q4_0: "q4_0", Q8_0: "q8_0", Q4_K: "q4_k", Q6_K: "q6_k", Q8_1: "q8_1",
             Q4_1: "q4_1", Q5_0: "q5_0", Q5_1: "q5_1", Q5_K: "q5_k"}

# fp16 scale ranges per format
D_RANGE = {Q4_0: (0.001, 0.02), Q8_0: (1e-4, 2e-3), Q4_K: (1e-4, 5e-3), Q6_K: (1e-4, 2e-3),
           Q4_1: (0.001, 0.02), Q5_0: (5e-4, 1e-2), Q5_1: (5e-4, 1e-2), Q5_K: (1e-4, 5e-3)}
DMIN_RANGE = (1e-4, 5e-3)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    wtype: int
    M: int
    K: int
    n: tuple
    n_experts: int = 0
    top_k: int = 0
    glu: bool = False

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def row_bytes(self) -> int:
        qk, bb = BLOCK[self.wtype]
        return self.K // qk * bb

    @property
    def weight_bytes(self) -> int:
        return self.M * self.row_bytes


WORKLOADS = [
    Workload(0, "q4_0_256x1024", Q4_0, 256, 1024, (1,)),
    Workload(1, "q4_k_4096x4096", Q4_K, 4096, 4096, (1,)),
    Workload(2, "q4_k_4096x14336", Q4_K, 4096, 14336, (1, 2, 4, 8)),
    Workload(3, "q6_k_128256x4096", Q6_K, 128256, 4096, (1,)),
    Workload(4, "moe_q4_k_8x14336x4096", Q4_K, 14336, 4096, (8,), n_experts=8, top_k=2,
             glu=True),
    # the other formats at the FFN-down shape (not among the reference configs)
    Workload(5, "q8_0_4096x14336", Q8_0, 4096, 14336, (1,)),
    Workload(6, "q4_1_4096x14336", Q4_1, 4096, 14336, (1,)),
    Workload(7, "q5_0_4096x14336", Q5_0, 4096, 14336, (1,)),
    Workload(8, "q5_1_4096x14336", Q5_1, 4096, 14336, (1,)),
    Workload(9, "q5_k_4096x14336", Q5_K, 4096, 14336, (1,)),
]
# The transposed FFN shape shares workload 2's seed and generator.
FFN_UP = Workload(2, "q4_k_14336x4096", Q4_K, 14336, 4096, (1, 2, 4, 8))
BY_NAME = {w.name: w for w in WORKLOADS + [FFN_UP]}


def streams(seed: int, count: int = 3):
    """Independent generators spawned from one seed (weights, x, ids)."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(count)]


def _fp16_bytes(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    v = rng.uniform(lo, hi, size=shape).astype(np.float32).astype(np.float16)
    return v.view(np.uint8).reshape(*shape, 2)


def weights(wtype: int, M: int, K: int, rng: np.random.Generator,
            d_range=None, dmin_range=None) -> np.ndarray:
    """Random weight matrix, uint8 array of shape [M, row_bytes]."""
    qk, bb = BLOCK[wtype]
    if K % qk:
        raise ValueError("K must be a multiple of the block size")
    nb = M * (K // qk)
    blk = np.empty((nb, bb), dtype=np.uint8)
    lo, hi = d_range or D_RANGE[wtype]
    if wtype == Q4_0:
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:18] = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    elif wtype == Q8_0:
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:34] = rng.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    elif wtype == Q4_K:
        mlo, mhi = dmin_range or DMIN_RANGE
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:4] = _fp16_bytes(rng, (nb,), mlo, mhi)
        blk[:, 4:144] = rng.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    elif wtype == Q6_K:
        blk[:, 0:192] = rng.integers(0, 256, size=(nb, 192), dtype=np.uint8)
        blk[:, 192:208] = rng.integers(-64, 64, size=(nb, 16), dtype=np.int8).view(np.uint8)
        blk[:, 208:210] = _fp16_bytes(rng, (nb,), lo, hi)
    elif wtype in (Q4_1, Q5_1):
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:4] = _fp16_bytes(rng, (nb,), -8.0 * hi, 0.0)
        blk[:, 4:bb] = rng.integers(0, 256, size=(nb, bb - 4), dtype=np.uint8)
    elif wtype == Q5_0:
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:22] = rng.integers(0, 256, size=(nb, 20), dtype=np.uint8)
    elif wtype == Q5_K:
        mlo, mhi = dmin_range or DMIN_RANGE
        blk[:, 0:2] = _fp16_bytes(rng, (nb,), lo, hi)
        blk[:, 2:4] = _fp16_bytes(rng, (nb,), mlo, mhi)
        blk[:, 4:176] = rng.integers(0, 256, size=(nb, 172), dtype=np.uint8)
    else:
        raise ValueError(f"unsupported weight type {wtype}")
    return blk.reshape(M, (K // qk) * bb)


def activations(K: int, n: int, rng: np.random.Generator, ldx: int | None = None) -> np.ndarray:
    """x ~ N(0, 1) float32, shape [n, ldx] (columns independent)."""
    ldx = K if ldx is None else ldx
    return rng.standard_normal(size=(n, ldx), dtype=np.float32)


def expert_ids(n_tokens: int, top_k: int, n_experts: int, rng: np.random.Generator) -> np.ndarray:
    """Per token, top_k distinct experts drawn uniformly without replacement
    (draw order kept). int32 [n_tokens, top_k]."""
    return np.stack([rng.choice(n_experts, size=top_k, replace=False)
                     for _ in range(n_tokens)]).astype(np.int32)


def make(workload: Workload, n: int | None = None):
    """Inputs of one workload: dict with W (or W_gate/W_up stacked over
    experts), x and ids."""
    rw, rx, ri = streams(workload.seed)
    n = workload.n[0] if n is None else n
    out = {"x": activations(workload.K, n, rx)}
    if workload.n_experts:
        E = workload.n_experts
        out["W_gate"] = np.stack([weights(workload.wtype, workload.M, workload.K, rw)
                                  for _ in range(E)])
        out["W_up"] = np.stack([weights(workload.wtype, workload.M, workload.K, rw)
                                for _ in range(E)])
        out["ids"] = expert_ids(n, workload.top_k, E, ri)
    else:
        out["W"] = weights(workload.wtype, workload.M, workload.K, rw)
    return out
