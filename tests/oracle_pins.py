"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix:

* hand-worked single-block examples under ``tests/golden/`` (derivations and
  citations inside each fixture);
* library routines the oracle's hand-written code must reduce to (numpy's
  IEEE binary16 conversion);
* the bit positions the pages' bit-level fragments fix (the Q4_K
  branch-free scale unpack and the Q6_K code assembly), restated here as
  fields of one wide little-endian integer and compared with the oracle's
  per-byte reading;
* brute force: fp64 dequantize-then-dot with dequantizers written here from
  the pages' row decoders, against the oracle's integer block dots;
* special cases that reduce to a plain integer dot, and invariants (column
  independence, the GLU composition, identity expert ids, zero padding,
  linearity in the block scale);
* the GLU variants at values the mathematics fixes (tabulated normal-CDF
  values for gelu, the swish identity, clamping) and the epilogue's order.

``test_oracle_pins.py`` runs them on the oracle as built;
``test_oracle_mutations.py`` runs them on copies of the oracle with planted
mistakes and requires each mistake to be caught.

Citations: [MMVQ §X] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时
一条量化权重如何被 dp4a 逐块点积", section X; [GGUF16 §X] = page "GGUF 量化内幕：
第16章 llama.cpp 量化代码架构", section X.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

Q4_0, Q8_0, Q8_1, Q4_K, Q6_K = 2, 8, 9, 12, 14
Q4_1, Q5_0, Q5_1, Q5_K = 3, 6, 7, 13
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def h2b(bits: str) -> bytes:
    return int(bits, 16).to_bytes(2, "little")


def q8_1_block(d_bits: str, s_bits: str, q) -> bytes:
    return h2b(d_bits) + h2b(s_bits) + np.asarray(q, dtype=np.int8).tobytes()


def f16(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------------------
# Dequantizers written here, from the pages, independent of the C oracle.
# ---------------------------------------------------------------------------

def _f16v(b: np.ndarray) -> np.ndarray:
    """little-endian fp16 from uint8 pairs -> float64"""
    return np.ascontiguousarray(b).view(np.float16).astype(np.float64).reshape(-1)


def deq_q4_0(row: np.ndarray, K: int) -> np.ndarray:
    """[MMVQ §权重的排法]: weight = d*(q-8); low nibbles are elements 0..15,
    high nibbles 16..31 (the pairing of qs words with activation words i and
    i+4 in [MMVQ §一次 vec_dot 的解剖])."""
    blk = row.reshape(K // 32, 18)
    d = _f16v(blk[:, 0:2])
    qs = blk[:, 2:18].astype(np.int64)
    codes = np.concatenate([qs & 15, qs >> 4], axis=1)
    return (d[:, None] * (codes - 8)).reshape(-1)


def deq_q8_0(row: np.ndarray, K: int) -> np.ndarray:
    """[LLM §量化格式]: 34 bytes per 32 weights, one fp16 scale and signed
    8-bit codes: weight = d*q."""
    blk = row.reshape(K // 32, 34)
    return (_f16v(blk[:, 0:2])[:, None] * blk[:, 2:34].view(np.int8).astype(np.float64)).reshape(-1)


def q4_k_scales_from_fragment(scales: np.ndarray):
    """Scales and mins of the 8 sub-blocks as bit fields of the 12 scale
    bytes read as one little-endian 96-bit integer V. The positions are
    worked out from the pages' branch-free unpack [MMVQ §一次 vec_dot 的解剖]
    (three 16-bit words, a mask selecting the first or second pair of
    sub-block pairs): sub-blocks 0-3 keep 6-bit fields in the low bits of
    bytes 0-3 (scales) and 4-7 (mins); sub-blocks 4-7 take their low 4 bits
    from a nibble of bytes 8-11 (scale: low nibble, min: high nibble) and
    their top 2 bits from the spare top bits of bytes 0-3 (scale) or 4-7
    (min). Written as (position, width) pairs, independent of the oracle's
    byte indexing."""
    V = int.from_bytes(bytes(np.asarray(scales, dtype=np.uint8)), "little")

    def bits(pos, width):
        return (V >> pos) & ((1 << width) - 1)

    sc, mn = [0] * 8, [0] * 8
    for t in range(8):
        if t < 4:
            sc[t] = bits(8 * t, 6)
            mn[t] = bits(32 + 8 * t, 6)
        else:
            k = t - 4
            sc[t] = bits(64 + 8 * k, 4) | bits(8 * k + 6, 2) << 4
            mn[t] = bits(64 + 8 * k + 4, 4) | bits(32 + 8 * k + 6, 2) << 4
    return sc, mn


def deq_q4_k(row: np.ndarray, K: int) -> np.ndarray:
    """[GGUF16 §16.2.1] row decoder: for each 64-element chunk c, sub-block
    2c takes the low nibbles of qs[32c..32c+31] and 2c+1 the high nibbles;
    weight = d*sc*q - dmin*m. Field order from the struct in [GGUF16 §16.1.2]."""
    out = []
    for blk in row.reshape(K // 256, 144):
        d = _f16v(blk[0:2])[0]
        dmin = _f16v(blk[2:4])[0]
        sc, mn = q4_k_scales_from_fragment(blk[4:16])
        qs = blk[16:144].astype(np.int64)
        for c in range(4):
            q = qs[32 * c:32 * c + 32]
            out.append(d * sc[2 * c] * (q & 15) - dmin * mn[2 * c])
            out.append(d * sc[2 * c + 1] * (q >> 4) - dmin * mn[2 * c + 1])
    return np.concatenate(out)


def q6_k_codes_from_fragment(blk: np.ndarray) -> np.ndarray:
    """Codes of one Q6_K block as bit fields of ql (128 bytes) and qh (64
    bytes), each read as one little-endian integer. The positions are worked
    out from the pages' code assembly [MMVQ §一次 vec_dot 的解剖]: a 32-bit
    word of ql gives four low-nibble codes or four high-nibble codes, and the
    matching word of qh, shifted by 0 or 2 for the first or second 32 bytes
    of a 64-byte ql half and by 4 more for the high nibbles, gives bits 4-5.
    So element e = 128h + 32g + l takes its low 4 bits at bit
    8(64h + 32(g mod 2) + l) + 4(g div 2) of ql and its top 2 bits at bit
    8(32h + l) + 2g of qh. Layout reading: ql[128] @0, qh[64] @128."""
    QL = int.from_bytes(bytes(blk[0:128]), "little")
    QH = int.from_bytes(bytes(blk[128:192]), "little")
    codes = np.zeros(256, dtype=np.int64)
    for e in range(256):
        h, g, l = e // 128, (e % 128) // 32, e % 32
        low = (QL >> (8 * (64 * h + 32 * (g % 2) + l) + 4 * (g // 2))) & 15
        high = (QH >> (8 * (32 * h + l) + 2 * g)) & 3
        codes[e] = low | high << 4
    return codes


def deq_q6_k(row: np.ndarray, K: int) -> np.ndarray:
    """weight = d*sc[e/16]*(q-32) with codes from the fragment above."""
    out = []
    for blk in row.reshape(K // 256, 210):
        codes = q6_k_codes_from_fragment(blk)
        sc = blk[192:208].view(np.int8).astype(np.float64)
        d = _f16v(blk[208:210])[0]
        out.append(d * np.repeat(sc, 16) * (codes - 32))
    return np.concatenate(out)


def _legacy_codes(qs: np.ndarray, qh=None) -> np.ndarray:
    """32 codes per block row: low nibbles are elements 0..15, high nibbles
    16..31 (as Q4_0); qh (4 bytes per block) adds bit e of its little-endian
    word as bit 4 of element e."""
    qs = qs.astype(np.int64)
    codes = np.concatenate([qs & 15, qs >> 4], axis=1)
    if qh is not None:
        word = (qh[:, 0].astype(np.int64) | (qh[:, 1].astype(np.int64) << 8) | (qh[:, 2].astype(np.int64) << 16)
                | (qh[:, 3].astype(np.int64) << 24))
        bits = (word[:, None] >> np.arange(32)[None, :]) & 1
        codes = codes + 16 * bits
    return codes


def deq_q4_1(row: np.ndarray, K: int) -> np.ndarray:
    """Reading of the GGUF Q4_1 block (the pages name the format): fp16 d @0,
    fp16 m @2, qs @4; weight = d*q + m."""
    blk = row.reshape(K // 32, 20)
    return (_f16v(blk[:, 0:2])[:, None] * _legacy_codes(blk[:, 4:20]) + _f16v(blk[:, 2:4])[:, None]).reshape(-1)


def deq_q5_0(row: np.ndarray, K: int) -> np.ndarray:
    """Reading of the GGUF Q5_0 block: fp16 d @0, qh @2, qs @6; weight =
    d*(q - 16)."""
    blk = row.reshape(K // 32, 22)
    return (_f16v(blk[:, 0:2])[:, None] * (_legacy_codes(blk[:, 6:22], blk[:, 2:6]) - 16)).reshape(-1)


def deq_q5_1(row: np.ndarray, K: int) -> np.ndarray:
    """Reading of the GGUF Q5_1 block: fp16 d @0, fp16 m @2, qh @4, qs @8;
    weight = d*q + m."""
    blk = row.reshape(K // 32, 24)
    return (_f16v(blk[:, 0:2])[:, None] * _legacy_codes(blk[:, 8:24], blk[:, 4:8])
            + _f16v(blk[:, 2:4])[:, None]).reshape(-1)


def deq_q5_k(row: np.ndarray, K: int) -> np.ndarray:
    """Reading of the GGUF Q5_K block: fp16 d @0, fp16 dmin @2, the Q4_K scale
    bytes @4, qh[32] @16, qs[128] @48. Element l of the low (high) nibble run
    of 64-element chunk c belongs to sub-block t = 2c (2c + 1) and takes bit t
    of qh[l] as bit 4; weight = d*sc_t*q - dmin*m_t."""
    out = []
    for blk in row.reshape(K // 256, 176):
        d = _f16v(blk[0:2])[0]
        dmin = _f16v(blk[2:4])[0]
        sc, mn = q4_k_scales_from_fragment(blk[4:16])
        qh = blk[16:48].astype(np.int64)
        qs = blk[48:176].astype(np.int64)
        for c in range(4):
            q = qs[32 * c:32 * c + 32]
            for h, t in ((0, 2 * c), (1, 2 * c + 1)):
                code = ((q >> (4 * h)) & 15) + 16 * ((qh >> t) & 1)
                out.append(d * sc[t] * code - dmin * mn[t])
    return np.concatenate(out)


DEQ = {Q4_0: deq_q4_0, Q8_0: deq_q8_0, Q4_K: deq_q4_k, Q6_K: deq_q6_k,
       Q4_1: deq_q4_1, Q5_0: deq_q5_0, Q5_1: deq_q5_1, Q5_K: deq_q5_k}
BLOCK = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210),
         Q4_1: (32, 20), Q5_0: (32, 22), Q5_1: (32, 24), Q5_K: (256, 176)}


def deq_y(col: np.ndarray, K: int) -> np.ndarray:
    b = col.reshape(K // 32, 36)
    return (_f16v(b[:, 0:2])[:, None] * b[:, 4:36].view(np.int8).astype(np.float64)).reshape(-1)


# ---------------------------------------------------------------------------
# Test-local encoders (inverse of the layouts read from the pages)
# ---------------------------------------------------------------------------

def pack_q4_0(d: float, codes) -> bytes:
    c = np.asarray(codes, dtype=np.uint8)
    return f16(d).tobytes() + (c[:16] | (c[16:] << 4)).astype(np.uint8).tobytes()


def pack_q4_k(d: float, dmin: float, scales12: bytes, codes) -> bytes:
    c = np.asarray(codes, dtype=np.uint8).reshape(4, 2, 32)   # chunk, parity, l
    qs = (c[:, 0, :] | (c[:, 1, :] << 4)).astype(np.uint8).reshape(-1)
    return f16(d).tobytes() + f16(dmin).tobytes() + bytes(scales12) + qs.tobytes()


def pack_q6_k(d: float, sc, codes) -> bytes:
    c = np.asarray(codes, dtype=np.int64).reshape(2, 4, 32)   # h, g, l
    ql = np.zeros(128, dtype=np.int64)
    qh = np.zeros(64, dtype=np.int64)
    for h in range(2):
        for g in range(4):
            low, high = c[h, g] & 15, c[h, g] >> 4
            base = 64 * h + 32 * (g % 2)
            ql[base:base + 32] |= low << (4 * (g // 2))
            qh[32 * h:32 * h + 32] |= high << (2 * g)
    return (ql.astype(np.uint8).tobytes() + qh.astype(np.uint8).tobytes()
            + np.asarray(sc, dtype=np.int8).tobytes() + f16(d).tobytes())


def q8_1_exact(qy: np.ndarray, d: float) -> np.ndarray:
    """q8_1 column from int8 codes with a chosen fp16 d; s = d*sum(q) is
    exactly representable in fp16 for the small sums used here."""
    qy = np.asarray(qy, dtype=np.int64).reshape(-1, 32)
    blocks = []
    for q in qy:
        s = float(f16(d)) * int(q.sum())
        assert float(f16(s)) == s, "choose d and codes so that s is exact"
        blocks.append(f16(d).tobytes() + f16(s).tobytes() + q.astype(np.int8).tobytes())
    return np.frombuffer(b"".join(blocks), dtype=np.uint8)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_type_info(O):
    """Block footprints [MMVQ §一次 vec_dot 的解剖 table; §激活的量化;
    GGUF16 §16.1.2; LLM §量化格式 (Q8_0 34 B/32)]: Q4_0 18 B/32, Q8_0 34 B/32,
    Q4_K 144 B/256, Q6_K 210 B/256, q8_1 36 B/32."""
    assert O.type_info(Q4_0) == (32, 18)
    assert O.type_info(Q8_0) == (32, 34)
    assert O.type_info(Q4_K) == (256, 144)
    assert O.type_info(Q6_K) == (256, 210)
    assert O.type_info(Q8_1) == (32, 36)
    # the formats the pages name without layouts: sizes of the GGUF blocks
    # (20, 22, 24 bytes per 32 weights; 176 per 256, ~5.5 bits a weight as
    # the LLM page's Q5_K_M row of ~22 B per 32 weights)
    assert O.type_info(Q4_1) == (32, 20)
    assert O.type_info(Q5_0) == (32, 22)
    assert O.type_info(Q5_1) == (32, 24)
    assert O.type_info(Q5_K) == (256, 176)


def pin_f16_decode(O):
    """Every binary16 bit pattern decodes as numpy does."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def f16_encode_cases(seed: int = 7) -> np.ndarray:
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-30, 17, size=20000)).astype(np.float32)
    signs = rng.choice([-1.0, 1.0], size=mags.size).astype(np.float32)
    # exact midpoints between neighbouring fp16 values (ties), normal and subnormal
    h = rng.integers(0, 0x7BFF, size=4000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2.0 ** -24,
                      2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11),
                      6.0975552e-05, 5.96e-08], dtype=np.float32)
    return np.concatenate([mags * signs, ties, -ties, edges])


def pin_f16_encode(O):
    """fp32 -> binary16 rounds to nearest even, as numpy does."""
    xs = f16_encode_cases()
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(v)) for v in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"first mismatch at {xs[bad[0]]!r}: {got[bad[0]]:#x} != {ref[bad[0]]:#x}"


def _check_q8_1_fixture(O, name):
    fx = golden(name)
    y = O.quantize_q8_1(np.asarray(fx["x"], dtype=np.float32).reshape(1, 32))[0]
    exp = fx["expected"]
    assert y[0:2].tobytes() == h2b(exp["d_bits"]), (name, y[0:2].tobytes().hex())
    assert y[2:4].tobytes() == h2b(exp["s_bits"]), (name, y[2:4].tobytes().hex())
    assert list(y[4:36].view(np.int8)) == exp["q"], name


def pin_q8_1_e1(O):
    _check_q8_1_fixture(O, "q8_1_e1.json")


def pin_q8_1_e2(O):
    _check_q8_1_fixture(O, "q8_1_e2.json")


def q8_1_property_inputs(seed: int = 11) -> np.ndarray:
    rng = np.random.default_rng(seed)
    blocks = []
    for scale in [1e-30, 1e-6, 1e-2, 1.0, 37.0, 1e4, 1e30]:
        blocks.append(rng.standard_normal((64, 32)).astype(np.float32) * np.float32(scale))
    z = np.zeros((4, 32), dtype=np.float32)
    z[1, 5] = 3.0            # one nonzero element
    z[2, :] = -2.0           # constant block
    z[3, ::2] = 1e-41        # subnormal inputs
    blocks.append(z)
    ties = (rng.integers(-100, 100, size=(16, 32)) + 0.5).astype(np.float32)
    ties[:, 0] = 127.0       # d = 1 exactly, so x/d hits the .5 ties
    blocks.append(ties)
    return np.concatenate(blocks).reshape(1, -1)


def pin_q8_1_properties(O):
    """q8_1 invariants [MMVQ §激活的量化]: |q| <= 127; the largest |x| of a
    nonzero block maps to |q| = 127; zero blocks give d = s = q = 0; the
    round trip is within half a step of the fp32 d plus the fp16 rounding
    of d; s rounds d*sum(q) (to within the fp16 rounding of d); rounding is
    to nearest with ties away from zero when d = 1."""
    x = q8_1_property_inputs()
    K = x.shape[1]
    y = O.quantize_q8_1(x).reshape(-1, 36)
    xb = x.reshape(-1, 32).astype(np.float64)
    d_h = y[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1)
    s_h = y[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)
    q = y[:, 4:36].view(np.int8).astype(np.int64)
    assert np.all(np.abs(q) <= 127)
    amax = np.abs(xb).max(axis=1)
    d32 = amax / 127.0                       # exact value; fp32 d is within 2^-24 of it
    for b in range(xb.shape[0]):
        if amax[b] == 0:
            assert d_h[b] == 0 and s_h[b] == 0 and not q[b].any()
            continue
        if d32[b] < 2.0 ** -126:             # d underflows: codes stay bounded only
            continue
        i = int(np.argmax(np.abs(xb[b])))
        assert abs(q[b, i]) == 127
        ulp16 = 2.0 ** (math.floor(math.log2(max(d32[b], 2.0 ** -14))) - 10)
        if d_h[b] > 0 and np.isfinite(d_h[b]):
            err = np.abs(xb[b] - d_h[b] * q[b])
            bound = (0.5 * d32[b] * (1 + 2.0 ** -20)
                     + np.abs(q[b]) * (0.5 * ulp16 + d32[b] * 2.0 ** -23))
            assert np.all(err <= bound + 1e-300), (b, err.max(), bound.max())
            sq = int(q[b].sum())
            if not np.isfinite(s_h[b]):      # d*sum(q) beyond the fp16 range
                assert abs(d32[b] * sq) >= 65504.0
                continue
            ds = abs(s_h[b] - d_h[b] * sq)
            s_ulp = 2.0 ** (math.floor(math.log2(max(abs(d32[b] * sq), 2.0 ** -14))) - 10) if sq else 0
            assert ds <= 0.5 * s_ulp + abs(sq) * (0.5 * ulp16 + d32[b] * 2.0 ** -23) + 1e-300
    # ties with d = 1: roundf semantics
    tb = xb[-16:]
    assert np.all(d_h[-16:] == 1.0)
    expect = np.sign(tb) * np.floor(np.abs(tb) + 0.5)
    assert np.array_equal(q[-16:], expect.astype(np.int64))
    assert K % 32 == 0


def _run_block(O, wtype, blk: bytes, ycol: np.ndarray, K: int):
    out, mag, dots = O.mmvq(np.frombuffer(blk, dtype=np.uint8), wtype, 1, K, ycol, 1,
                            want_dots=True)
    return out[0, 0], mag[0, 0], dots[0, 0]


def pin_q4_0_e3(O):
    fx = golden("q4_0_e3.json")
    blk = bytes.fromhex(fx["weight_block_hex"])
    yb = fx["q8_1_block"]
    y = np.frombuffer(q8_1_block(yb["d_bits"], yb["s_bits"], yb["q"]), dtype=np.uint8)
    out, mag, dots = _run_block(O, Q4_0, blk, y, 32)
    e = fx["expected"]
    assert dots[0][0] == e["isum"] and out == e["out"] and mag == e["mag"], (dots, out, mag)


def pin_q8_0_e6(O):
    fx = golden("q8_0_e6.json")
    blk = bytes.fromhex(fx["weight_block_hex"])
    yb = fx["q8_1_block"]
    y = np.frombuffer(q8_1_block(yb["d_bits"], yb["s_bits"], yb["q"]), dtype=np.uint8)
    out, mag, dots = _run_block(O, Q8_0, blk, y, 32)
    e = fx["expected"]
    assert dots[0][0] == e["isum"] and out == e["out"] and mag == e["mag"], (dots, out, mag)


def _pin_legacy_golden(O, fname, wtype):
    fx = golden(fname)
    blk = bytes.fromhex(fx["weight_block_hex"])
    yb = fx["q8_1_block"]
    y = np.frombuffer(q8_1_block(yb["d_bits"], yb["s_bits"], yb["q"]), dtype=np.uint8)
    out, mag, dots = _run_block(O, wtype, blk, y, 32)
    e = fx["expected"]
    assert dots[0][0] == e["isum"] and out == e["out"] and mag == e["mag"], (fname, dots, out, mag)


def pin_q4_1_e7(O):
    _pin_legacy_golden(O, "q4_1_e7.json", Q4_1)


def pin_q5_0_e8(O):
    _pin_legacy_golden(O, "q5_0_e8.json", Q5_0)


def pin_q5_1_e9(O):
    _pin_legacy_golden(O, "q5_1_e9.json", Q5_1)


def pin_q5_k_e10(O):
    fx = golden("q5_k_e10.json")
    hdr = bytes.fromhex(fx["weight_block_header_hex"])
    blk = hdr + bytes([int(fx["qh_byte"], 16)]) * 32 + bytes([int(fx["qs_byte"], 16)]) * 128
    y = np.frombuffer(b"".join(q8_1_block(b["d_bits"], b["s_bits"], [b["q_all"]] * 32) for b in fx["q8_1_blocks"]),
                      dtype=np.uint8)
    out, mag, dots = _run_block(O, Q5_K, blk, y, 256)
    e = fx["expected"]
    assert list(dots[0][:8]) == e["dot1"] and list(dots[0][8:]) == e["dot2"], dots
    assert out == e["out"] and mag == e["mag"], (out, mag)


def pin_q4_k_e4(O):
    fx = golden("q4_k_e4.json")
    hdr = bytes.fromhex(fx["weight_block_header_hex"])
    blk = hdr + bytes([int(fx["qs_byte"], 16)]) * 128
    yb = fx["q8_1_blocks"]
    y = np.frombuffer(q8_1_block(yb["d_bits"], yb["s_bits"], [yb["q_all"]] * 32) * yb["count"],
                      dtype=np.uint8)
    out, mag, dots = _run_block(O, Q4_K, blk, y, 256)
    e = fx["expected"]
    scales = hdr[4:16]
    assert [O.q4_k_scale_min(scales, t) for t in range(8)] == list(zip(e["sc"], e["m"]))
    assert list(dots[0][:8]) == e["dot1"] and list(dots[0][8:]) == e["dot2"], dots
    assert out == e["out"] and mag == e["mag"], (out, mag)


def pin_k_min_magnitude_halves(O):
    """The tolerance's error scale for Q4_K and Q5_K sums both terms over each
    16-element half of a sub-block (an fp32 evaluation may scale the halves'
    partial dots before they meet). Hand-worked block: d = 1, dmin = 0,
    sc = 1 and m = 0 for all 8 sub-blocks (scale bytes 01 01 01 01 00 00 00 00
    01 01 01 01 by the 6-bit packing: sub-blocks 0-3 take the low 6 bits of
    bytes 0-3 and 4-7, sub-blocks 4-7 the nibbles of bytes 8-11), every code
    1 (qs bytes 0x11; Q5_K: qh bytes 0, so the fifth bits are 0), and q8_1
    blocks with d8 = 1, qy = +1 on elements 0-15 and -1 on 16-31. Each half
    dot is +16 or -16 and each sub-block's dot 0: the result is 0, the
    magnitude 8 sub-blocks x 2 halves x 16 = 256 (it would be 0 over whole
    sub-blocks)."""
    hdr = h2b("0x3C00") + h2b("0x0000") + bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])
    y = np.frombuffer(q8_1_block("0x3C00", "0x0000", [1] * 16 + [-1] * 16) * 8, dtype=np.uint8)
    for wtype, blk in ((Q4_K, hdr + bytes([0x11]) * 128), (Q5_K, hdr + bytes(32) + bytes([0x11]) * 128)):
        out, mag, dots = _run_block(O, wtype, blk, y, 256)
        assert list(dots[0][:8]) == [0] * 8 and list(dots[0][8:]) == [0] * 8, dots
        assert out == 0.0 and mag == 256.0, (wtype, out, mag)


def pin_q6_k_e5(O):
    fx = golden("q6_k_e5.json")
    ql = bytearray(bytes.fromhex(fx["ql_hex_default"]) * 128)
    for k, v in fx["ql_overrides"].items():
        ql[int(k)] = int(v, 16)
    qh = bytearray(bytes.fromhex(fx["qh_hex_default"]) * 64)
    for k, v in fx["qh_overrides"].items():
        qh[int(k)] = int(v, 16)
    blk = bytes(ql) + bytes(qh) + np.asarray(fx["sc"], dtype=np.int8).tobytes() + h2b(fx["d_bits"])
    yb = fx["q8_1_blocks"]
    y = np.frombuffer(q8_1_block(yb["d_bits"], yb["s_bits"], [yb["q_all"]] * 32) * yb["count"],
                      dtype=np.uint8)
    out, mag, dots = _run_block(O, Q6_K, blk, y, 256)
    e = fx["expected"]
    w = O.dequantize_row(Q6_K, np.frombuffer(blk, dtype=np.uint8), 256)
    # sc = 1..16, d = 1: w = sc*(q-32), so the codes are recoverable
    codes = w / np.repeat(np.arange(1, 17), 16) + 32
    assert codes[100] == e["code_e100"] and codes[200] == e["code_e200"]
    assert np.count_nonzero(codes != 32) == 2
    assert out == e["out"] and mag == e["mag"], (out, mag)


def pin_q4_k_fragment(O, seed: int = 3):
    """The oracle's per-sub-block unpack equals the bit positions read from
    the pages' branch-free fragment, on random scale bytes."""
    rng = np.random.default_rng(seed)
    for _ in range(400):
        s = rng.integers(0, 256, size=12, dtype=np.uint8)
        sc, mn = q4_k_scales_from_fragment(s)
        got = [O.q4_k_scale_min(s.tobytes(), t) for t in range(8)]
        assert got == list(zip(sc, mn)), (s.tobytes().hex(), got, sc, mn)


def pin_q4_k_bijection(O, seed: int = 5):
    """The 8 scales and 8 mins use all 96 bits of the 12 bytes once: flipping
    any one bit changes exactly one 6-bit field by a power of two."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 256, size=12, dtype=np.uint8)
    base = [v for t in range(8) for v in O.q4_k_scale_min(s.tobytes(), t)]
    hit = set()
    for byte in range(12):
        for bit in range(8):
            s2 = s.copy()
            s2[byte] ^= 1 << bit
            now = [v for t in range(8) for v in O.q4_k_scale_min(s2.tobytes(), t)]
            diff = [i for i in range(16) if now[i] != base[i]]
            assert len(diff) == 1, (byte, bit, diff)
            delta = abs(now[diff[0]] - base[diff[0]])
            assert delta & (delta - 1) == 0 and delta < 64
            hit.add((diff[0], delta))
    assert len(hit) == 96


def pin_q6_k_fragment(O, seed: int = 9):
    """Codes from the oracle's per-element reading equal the bit positions
    read from the pages' 32-bit code assembly."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        blk = bytearray(rng.integers(0, 256, size=210, dtype=np.uint8).tobytes())
        blk[192:208] = bytes([1] * 16)
        blk[208:210] = f16(1.0).tobytes()
        blk = np.frombuffer(bytes(blk), dtype=np.uint8)
        w = O.dequantize_row(Q6_K, blk, 256)
        assert np.array_equal(w + 32, q6_k_codes_from_fragment(blk).astype(np.float64))


def _tiny(wtype, M, K, seed):
    from quantized_decode_gemv_quantize_amd import synth
    rng = np.random.default_rng(seed)
    W = synth.weights(wtype, M, K, rng)
    x = rng.standard_normal((2, K)).astype(np.float32)
    return W, x


def pin_brute_force(O, seeds=(0, 1, 2)):
    """Integer block dots with scales applied afterwards equal fp64
    dequantize-then-dot [MMVQ §一次 vec_dot 的解剖; GGUF16 §16.2.2]. K-quants
    agree to fp64 roundoff; Q4_0 uses the fp16 s, so it agrees to within
    8*|d_w|*|s - d8*sum(q)| per block."""
    for wtype, Ks in [(Q4_0, (32, 64, 256)), (Q8_0, (32, 96)), (Q4_K, (256, 512)), (Q6_K, (256, 512)),
                      (Q4_1, (32, 96)), (Q5_0, (32, 96)), (Q5_1, (32, 96)), (Q5_K, (256, 512))]:
        qk, bb = BLOCK[wtype]
        for K in Ks:
            for seed in seeds:
                M = 3
                W, x = _tiny(wtype, M, K, 100 * wtype + 7 * K + seed)
                y = O.quantize_q8_1(x)
                out, mag, _ = O.mmvq(W, wtype, M, K, y, 2)
                for j in range(2):
                    yd = deq_y(y[j], K)
                    for r in range(M):
                        w = DEQ[wtype](W[r], K)
                        assert np.array_equal(w, O.dequantize_row(wtype, W[r], K)), (wtype, K, r)
                        ref = float(np.dot(w, yd))
                        if wtype in (Q4_0, Q4_1, Q5_0, Q5_1):
                            # the old-style formats take the offset term from
                            # the fp16 s: off by |offset| * |s - d8*sum(q)|
                            yb = y[j].reshape(-1, 36)
                            d8 = yb[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1)
                            s8 = yb[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)
                            sq = yb[:, 4:36].view(np.int8).astype(np.int64).sum(axis=1)
                            wb = W[r].reshape(-1, bb)
                            dw = np.abs(wb[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(-1))
                            off = {Q4_0: 8 * dw, Q5_0: 16 * dw}.get(
                                wtype, np.abs(wb[:, 2:4].copy().view(np.float16).astype(np.float64).reshape(-1)))
                            tol = float(np.sum(off * np.abs(s8 - d8 * sq))) * (1 + 1e-9) + 1e-12
                        else:
                            tol = 1e-12 * mag[j, r] + 1e-15
                        assert abs(out[j, r] - ref) <= tol, (wtype, K, seed, j, r, out[j, r], ref)


def pin_int_dot_special(O, seed: int = 21):
    """With unit scales and no min the product is a plain integer dot of the
    codes (minus the zero point) with the activation codes [MMVQ §dp4a]."""
    rng = np.random.default_rng(seed)
    for K in (256, 512):
        qy = rng.integers(-3, 4, size=K)
        y = q8_1_exact(qy, 0.5)
        # Q4_0: d = 1, weight q-8
        codes = rng.integers(0, 16, size=K)
        W = b"".join(pack_q4_0(1.0, codes[32 * b:32 * b + 32]) for b in range(K // 32))
        out, _, _ = O.mmvq(W, Q4_0, 1, K, y, 1)
        assert out[0, 0] == 0.5 * float(np.dot(codes - 8, qy))
        # Q4_K: d = 1, dmin = 0, every sc = 1 and m = 0
        scales = bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])
        W = b"".join(pack_q4_k(1.0, 0.0, scales, codes[256 * b:256 * b + 256])
                     for b in range(K // 256))
        out, _, _ = O.mmvq(W, Q4_K, 1, K, y, 1)
        assert out[0, 0] == 0.5 * float(np.dot(codes, qy))
        # Q4_K min only: codes 0, m = 1 everywhere -> -dmin * sum(d8*qy)
        scales_m = bytes([0, 0, 0, 0, 1, 1, 1, 1, 0x10, 0x10, 0x10, 0x10])
        W = b"".join(pack_q4_k(1.0, 2.0, scales_m, np.zeros(256, dtype=int)) for _ in range(K // 256))
        out, _, _ = O.mmvq(W, Q4_K, 1, K, y, 1)
        assert out[0, 0] == -2.0 * 0.5 * float(qy.sum())
        # Q6_K: d = 1, every sc = 1, weight q-32
        c6 = rng.integers(0, 64, size=K)
        W = b"".join(pack_q6_k(1.0, [1] * 16, c6[256 * b:256 * b + 256]) for b in range(K // 256))
        out, _, _ = O.mmvq(W, Q6_K, 1, K, y, 1)
        assert out[0, 0] == 0.5 * float(np.dot(c6 - 32, qy))
        # Q8_0: d = 1, weight q (signed, no zero point)
        c8 = rng.integers(-127, 128, size=K)
        W = b"".join(f16(1.0).tobytes() + c8[32 * b:32 * b + 32].astype(np.int8).tobytes()
                     for b in range(K // 32))
        out, _, _ = O.mmvq(W, Q8_0, 1, K, y, 1)
        assert out[0, 0] == 0.5 * float(np.dot(c8, qy))


def pin_columns_independent(O, seed: int = 31):
    """n activation columns give n independent products [MMVQ §多个 token 时]."""
    for wtype, K in [(Q4_0, 256), (Q4_K, 512), (Q6_K, 512)]:
        W, x = _tiny(wtype, 5, K, seed + wtype)
        x3 = np.concatenate([x, x[:1] * 2])
        y = O.quantize_q8_1(x3)
        out, mag, _ = O.mmvq(W, wtype, 5, K, y, 3)
        for j in range(3):
            o1, m1, _ = O.mmvq(W, wtype, 5, K, y[j:j + 1], 1)
            assert np.array_equal(out[j], o1[0]) and np.array_equal(mag[j], m1[0])


def pin_glu(O, seed: int = 41):
    """Fused gate/up equals the composition GLU(W_gate.y, W_up.y) through the
    one GLU routine the epilogue forms use [MMVQ §融合], for every op that
    takes no caller parameter; the clamp op, which needs a limit, is refused
    here; a zero gate gives zero output (silu, gelu and the OAI form vanish
    at 0)."""
    from oracle import OracleError
    for wtype, K in [(Q4_0, 256), (Q4_K, 512), (Q6_K, 256)]:
        Wg, x = _tiny(wtype, 4, K, seed + wtype)
        Wu, _ = _tiny(wtype, 4, K, seed + wtype + 1)
        y = O.quantize_q8_1(x)
        g, _, _ = O.mmvq(Wg, wtype, 4, K, y, 2)
        u, _, _ = O.mmvq(Wu, wtype, 4, K, y, 2)
        for op in (0, 1, GEGLU, SWIGLU_OAI):
            got = O.mmvq_glu(Wg, Wu, wtype, 4, K, y, 2, op)
            ref = np.array([[O.glu(op, g[j, r], u[j, r]) for r in range(4)] for j in range(2)])
            assert np.array_equal(got, ref)
        try:
            O.mmvq_glu(Wg, Wu, wtype, 4, K, y, 2, SWIGLU_CLAMP)
        except OracleError as err:
            assert err.code == -2
        else:
            raise AssertionError("clamp op accepted without a limit")
    # zero gate: d = 0 in every gate block
    qk, bb = BLOCK[Q4_0]
    Wg, x = _tiny(Q4_0, 2, 64, 1)
    Wg = Wg.copy().reshape(-1, bb)
    Wg[:, 0:2] = 0
    Wu, _ = _tiny(Q4_0, 2, 64, 2)
    y = O.quantize_q8_1(x)
    for op in (0, 1, GEGLU, SWIGLU_OAI):
        assert not O.mmvq_glu(Wg.reshape(-1), Wu, Q4_0, 2, 64, y, 2, op).any()


def pin_id(O, seed: int = 51):
    """Expert-indexed product [MMVQ §MoE]: each (token, slot) output is the
    chosen expert's rows against that token's column; identity ids reduce
    to per-expert products; out-of-range ids are rejected."""
    from quantized_decode_gemv_quantize_amd import synth
    rng = np.random.default_rng(seed)
    for wtype, K in [(Q4_K, 256), (Q4_0, 64), (Q6_K, 256)]:
        E, M, T, top_k = 4, 3, 3, 2
        Ws = [synth.weights(wtype, M, K, rng) for _ in range(E)]
        W = np.concatenate([w.reshape(-1) for w in Ws])
        stride = Ws[0].size
        x = rng.standard_normal((T, K)).astype(np.float32)
        y = O.quantize_q8_1(x)
        ids = np.array([[2, 0], [1, 3], [3, 2]], dtype=np.int32)
        out, mag = O.mmvq_id(W, stride, E, wtype, M, K, y, T, ids, top_k)
        for t in range(T):
            for k in range(top_k):
                ref, rmag, _ = O.mmvq(Ws[ids[t, k]], wtype, M, K, y[t:t + 1], 1)
                assert np.array_equal(out[t * top_k + k], ref[0])
                assert np.array_equal(mag[t * top_k + k], rmag[0])
        ident = np.arange(T, dtype=np.int32).reshape(T, 1)
        out1, _ = O.mmvq_id(W, stride, E, wtype, M, K, y, T, ident, 1)
        for t in range(T):
            ref, _, _ = O.mmvq(Ws[t], wtype, M, K, y[t:t + 1], 1)
            assert np.array_equal(out1[t], ref[0])
        Wu = np.concatenate([synth.weights(wtype, M, K, rng).reshape(-1) for _ in range(E)])
        og = O.mmvq_id_glu(W, Wu, stride, E, wtype, M, K, y, T, ids, top_k, 1)
        for t in range(T):
            for k in range(top_k):
                e = int(ids[t, k])
                ref = O.mmvq_glu(Ws[e], Wu[e * stride:(e + 1) * stride], wtype, M, K,
                                 y[t:t + 1], 1, 1)
                assert np.array_equal(og[t * top_k + k], ref[0])
        from oracle import OracleError
        try:
            O.mmvq_id(W, stride, E, wtype, M, K, y, T, np.array([[0, 4]] * T, dtype=np.int32), 2)
        except OracleError as e:
            assert e.code == -6
        else:
            raise AssertionError("out-of-range id accepted")


def pin_zero_padding(O, seed: int = 61):
    """Zero activations appended to K leave the product unchanged, whatever
    the weights there [MMVQ §激活的量化 (padding quantizes to 0)]."""
    from quantized_decode_gemv_quantize_amd import synth
    rng = np.random.default_rng(seed)
    for wtype, K, P in [(Q4_0, 64, 64), (Q8_0, 64, 32), (Q4_K, 256, 256), (Q6_K, 256, 256)]:
        W = synth.weights(wtype, 3, K + P, rng)
        x = np.zeros((1, K + P), dtype=np.float32)
        x[0, :K] = rng.standard_normal(K)
        y = O.quantize_q8_1(x)
        qk, bb = BLOCK[wtype]
        Wk = np.ascontiguousarray(W[:, :(K // qk) * bb])
        a, _, _ = O.mmvq(W, wtype, 3, K + P, y, 1)
        b, _, _ = O.mmvq(Wk, wtype, 3, K, np.ascontiguousarray(y[:, :(K // 32) * 36]), 1)
        assert np.array_equal(a, b)


def pin_linearity(O, seed: int = 71):
    """Doubling every weight block scale (exact in fp16) doubles the output."""
    from quantized_decode_gemv_quantize_amd import synth
    rng = np.random.default_rng(seed)
    for wtype, K, fields in [(Q4_0, 128, [(0, 2)]), (Q8_0, 64, [(0, 2)]), (Q4_K, 256, [(0, 2), (2, 4)]),
                             (Q6_K, 256, [(208, 210)])]:
        W = synth.weights(wtype, 2, K, rng)
        y = O.quantize_q8_1(rng.standard_normal((1, K)).astype(np.float32))
        W2 = W.copy().reshape(-1, BLOCK[wtype][1])
        for a, b in fields:
            v = W2[:, a:b].copy().view(np.float16)
            W2[:, a:b] = (v * np.float16(2)).view(np.uint8)
        o1, _, _ = O.mmvq(W, wtype, 2, K, y, 1)
        o2, _, _ = O.mmvq(W2.reshape(-1), wtype, 2, K, y, 1)
        assert np.allclose(o2, 2 * o1, rtol=1e-15, atol=0)


# Standard normal CDF Phi(z), printed-table constants (not computed here).
NORMAL_CDF = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208,
              3.0: 0.9986501019683699}
GEGLU, SWIGLU_OAI, SWIGLU_CLAMP = 2, 3, 4
# Constants of the published forms the GLU readings take (parity unpinned
# against the pages, which print none of these formulas): the tanh form of
# GELU (Hendrycks and Gimpel, 2016) and the clamped SwiGLU of the gpt-oss
# models (alpha 1.702, limit 7).
GELU_C, GELU_A = math.sqrt(2.0 / math.pi), 0.044715
OAI_ALPHA, OAI_LIMIT = 1.702, 7.0


def pin_glu_variants(O):
    """GLU ops of the fused epilogue [MMVQ §融合] at values fixed by the
    mathematics and by the sources the readings name (the pages fix none):
    * silu: sigmoid(ln 3) = 3/4 and sigmoid(ln 2) = 2/3 exactly, so
      silu(ln 3) = (3/4) ln 3 and silu(ln 2) = (2/3) ln 2; s(z) - s(-z) = z;
    * gelu (tanh form): g(z) - g(-z) = z; atanh(2 g(z)/z - 1) / z is the
      line c + c*a*z^2 in z^2 with the published c = sqrt(2/pi),
      a = 0.044715 (an erf gelu is not of that shape); within 1e-3*|z| of
      z*Phi(z) at tabulated normal-CDF values, and not equal to it;
    * OAI: at g = ln(3)/1.702 the sigmoid is 3/4, so out = (3/4) g (u'+1);
      the swish identity with (u'+1); the gate clamps at +7 from above only,
      the up value at +-7;
    * clamp: silu on clamped values with the caller's limit;
    plain is g*u; an unknown op is rejected."""
    from oracle import OracleError
    for z, s in ((math.log(3.0), 0.75), (math.log(2.0), 2.0 / 3.0)):
        for u in (1.0, -2.5):
            assert abs(O.glu(1, z, u) - s * z * u) <= 2e-15 * abs(z * u)
    for z in (0.5, 1.0, 1.5, 2.5):
        gz = O.glu(GEGLU, z, 1.0)
        assert abs(gz - O.glu(GEGLU, -z, 1.0) - z) <= 1e-14 * z
        h = math.atanh(2.0 * gz / z - 1.0) / z
        assert abs(h - (GELU_C + GELU_C * GELU_A * z * z)) <= 1e-12
    for z, phi in NORMAL_CDF.items():
        d = abs(O.glu(GEGLU, z, 1.0) - z * phi)
        assert d <= 1e-3 * z and d > 1e-7 * z
        assert abs(O.glu(GEGLU, z, -3.0) + 3.0 * O.glu(GEGLU, z, 1.0)) <= 1e-14 * z
    assert O.glu(GEGLU, 0.0, 5.0) == 0.0
    g34 = math.log(3.0) / OAI_ALPHA
    for u in (-9.0, -2.0, 0.5, 3.0, 20.0):
        uc = min(max(u, -OAI_LIMIT), OAI_LIMIT)
        assert abs(O.glu(SWIGLU_OAI, g34, u) - 0.75 * g34 * (uc + 1.0)) <= 4e-15 * (1 + abs(uc + 1))
    L = 3.0
    for g in (0.25, 1.0, 2.9, 6.9):
        for u in (-9.0, -2.0, 0.5, 3.0, 20.0):
            uc = min(max(u, -OAI_LIMIT), OAI_LIMIT)
            ul = min(max(u, -L), L)
            assert abs(O.glu(1, g, u) - O.glu(1, -g, u) - g * u) <= 1e-13 * (1 + abs(g * u))
            dd = O.glu(SWIGLU_OAI, g, u) - O.glu(SWIGLU_OAI, -g, u)
            assert abs(dd - g * (uc + 1.0)) <= 1e-13 * (1 + abs(g * (uc + 1)))
            assert O.glu(SWIGLU_OAI, g, u) == O.glu(SWIGLU_OAI, g, uc)
            assert O.glu(SWIGLU_CLAMP, g, u, L) == O.glu(SWIGLU_CLAMP, min(g, L), ul, L)
            if g <= L and -L <= u <= L:
                assert O.glu(SWIGLU_CLAMP, g, u, L) == O.glu(1, g, u)
            assert O.glu(0, g, u) == g * u
    for u in (-3.0, 0.0, 2.0):
        assert O.glu(SWIGLU_OAI, 50.0, u) == O.glu(SWIGLU_OAI, OAI_LIMIT, u)
        assert O.glu(SWIGLU_OAI, 50.0, u) != O.glu(SWIGLU_OAI, 6.0, u) or u == -1.0
        assert O.glu(SWIGLU_CLAMP, 50.0, u, L) == O.glu(SWIGLU_CLAMP, L, u, L)
        assert O.glu(SWIGLU_OAI, 0.0, u) == 0.0
    # the gates are clamped from above only: a very negative gate is not lifted
    assert O.glu(SWIGLU_CLAMP, -20.0, 1.0, L) != O.glu(SWIGLU_CLAMP, -L, 1.0, L)
    assert O.glu(SWIGLU_OAI, -20.0, 1.0) != O.glu(SWIGLU_OAI, -OAI_LIMIT, 1.0)
    # the OAI limit is the op's own: the caller's limit argument does not move it
    assert O.glu(SWIGLU_OAI, 6.5, 1.0, 2.0) == O.glu(SWIGLU_OAI, 6.5, 1.0, 50.0)
    try:
        O.glu(9, 1.0, 1.0)
    except OracleError as e:
        assert e.code == -2
    else:
        raise AssertionError("unknown glu op accepted")


def pin_epilogue(O, seed: int = 81):
    """The full epilogue in the pages' order [MMVQ §融合]: up result times its
    scale, plus its bias row; the same for the gate; then the GLU. With no
    epilogue and no gate it is the plain product; the expert-indexed form
    uses each slot's expert scale and bias row; the shared expert is the
    plain GLU product of the shared matrices for every token."""
    from quantized_decode_gemv_quantize_amd import synth
    rng = np.random.default_rng(seed)
    for wtype, K in [(Q4_K, 512), (Q4_0, 128), (Q6_K, 256)]:
        M = 5
        Wu, x = _tiny(wtype, M, K, seed + wtype)
        Wg, _ = _tiny(wtype, M, K, seed + wtype + 1)
        y = O.quantize_q8_1(x)
        u, _, _ = O.mmvq(Wu, wtype, M, K, y, 2)
        g, _, _ = O.mmvq(Wg, wtype, M, K, y, 2)
        assert np.array_equal(O.mmvq_ex(Wu, None, wtype, M, K, y, 2), u)
        ub, gb = rng.standard_normal(M), rng.standard_normal(M)
        out = O.mmvq_ex(Wu, None, wtype, M, K, y, 2, dict(up_bias=ub, up_scale=[0.75]))
        assert np.allclose(out, u * 0.75 + ub, rtol=1e-15, atol=1e-15)
        for op in range(5):
            epi = dict(up_bias=ub, gate_bias=gb, up_scale=[1.25], gate_scale=[-0.5], glu_op=op,
                       limit=2.0)
            out = O.mmvq_ex(Wu, Wg, wtype, M, K, y, 2, epi)
            for j in range(2):
                for r in range(M):
                    ref = O.glu(op, g[j, r] * -0.5 + gb[r], u[j, r] * 1.25 + ub[r], 2.0)
                    assert abs(out[j, r] - ref) <= 1e-14 * (1 + abs(ref))
        # expert-indexed form with per-expert scales and bias rows, and a shared expert
        E, T, top_k = 3, 2, 2
        Ws = [synth.weights(wtype, M, K, rng) for _ in range(2 * E)]
        stride = Ws[0].size
        Wu_all = np.concatenate([w.reshape(-1) for w in Ws[:E]])
        Wg_all = np.concatenate([w.reshape(-1) for w in Ws[E:]])
        Su, Sg = synth.weights(wtype, M, K, rng), synth.weights(wtype, M, K, rng)
        ids = np.array([[2, 0], [1, 2]], dtype=np.int32)
        sc_u, sc_g = rng.uniform(0.5, 2.0, E), rng.uniform(0.5, 2.0, E)
        b_u, b_g = rng.standard_normal(E * M), rng.standard_normal(E * M)
        epi = dict(up_bias=b_u, gate_bias=b_g, up_scale=sc_u, gate_scale=sc_g, glu_op=1)
        out, sh = O.mmvq_id_ex(Wu_all, Wg_all, stride, E, wtype, M, K, y, T, ids, top_k, epi, Su, Sg)
        for t in range(T):
            for k in range(top_k):
                e = int(ids[t, k])
                one = dict(up_bias=b_u[e * M:(e + 1) * M], gate_bias=b_g[e * M:(e + 1) * M],
                           up_scale=[sc_u[e]], gate_scale=[sc_g[e]], glu_op=1)
                ref = O.mmvq_ex(Ws[e], Ws[E + e], wtype, M, K, y[t:t + 1], 1, one)
                assert np.array_equal(out[t * top_k + k], ref[0])
            ref = O.mmvq_ex(Su, Sg, wtype, M, K, y[t:t + 1], 1, dict(glu_op=1))
            assert np.array_equal(sh[t], ref[0])


def pin_error_codes(O):
    """Bad arguments return codes instead of aborting."""
    L = O.L
    assert L.orc_mmvq(None, Q4_K, 1, 256, None, 1, None, None, None) == -1
    buf = np.zeros(4096, dtype=np.uint8)
    p = buf.ctypes.data
    assert L.orc_mmvq(p, 5, 1, 256, p, 1, p, None, None) == -2   # id 5: removed from the enumeration
    assert L.orc_mmvq(p, Q4_K, 1, 200, p, 1, p, None, None) == -3
    assert L.orc_mmvq(p, Q4_K, 0, 256, p, 1, p, None, None) == -3
    assert L.orc_quantize_q8_1(p, 33, 1, 33, p) == -3
    assert L.orc_quantize_q8_1(p, 32, 1, 16, p) == -3


ALL_PINS = [pin_type_info, pin_f16_decode, pin_f16_encode, pin_q8_1_e1, pin_q8_1_e2,
            pin_q8_1_properties, pin_q4_0_e3, pin_q4_k_e4, pin_q6_k_e5, pin_q8_0_e6, pin_q4_1_e7,
            pin_q5_0_e8, pin_q5_1_e9, pin_q5_k_e10, pin_q4_k_fragment,
            pin_q4_k_bijection, pin_q6_k_fragment, pin_brute_force, pin_int_dot_special,
            pin_columns_independent, pin_glu, pin_id, pin_zero_padding, pin_linearity,
            pin_glu_variants, pin_epilogue, pin_error_codes, pin_k_min_magnitude_halves]
