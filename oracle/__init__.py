"""CPU oracle for the decode-time quantized mat-vec (MMVQ).

TEST INFRASTRUCTURE ONLY. This package wraps ``libmmvq_oracle.so`` (plain C,
fp64 accumulation, built from ``mmvq_oracle.c`` with gcc). Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it. The product library and its Python binding never import it, and
the two share no code: only the seeded input generator
(``quantized_decode_gemv_quantize_amd.synth``) feeds both.

What each function computes is stated in ``mmvq_oracle.h``; the page
citations are there and in ``mmvq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mmvq_oracle.c")
LIB = os.path.join(HERE, "libmmvq_oracle.so")

Q4_0, Q8_0, Q8_1, Q4_K, Q6_K = 2, 8, 9, 12, 14
Q4_1, Q5_0, Q5_1, Q5_K = 3, 6, 7, 13
GLU_PLAIN, GLU_SWIGLU, GLU_GEGLU, GLU_SWIGLU_OAI, GLU_SWIGLU_CLAMP = 0, 1, 2, 3, 4
BLOCK = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210), Q8_1: (32, 36),
         Q4_1: (32, 20), Q5_0: (32, 22), Q5_1: (32, 24), Q5_K: (256, 176)}
DOTS_PER_BLOCK = {Q4_0: 1, Q8_0: 1, Q4_K: 16, Q6_K: 16, Q4_1: 1, Q5_0: 1, Q5_1: 1, Q5_K: 16}

_c_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, no fp contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
            "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle returned {code}")
        self.code = code


def _check(rc: int) -> None:
    if rc != 0:
        raise OracleError(rc)


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.frombuffer(a, dtype=np.uint8) if isinstance(a, (bytes, bytearray))
                                else a).view(np.uint8).reshape(-1)


class _Epilogue(ctypes.Structure):
    _fields_ = [("up_bias", _p), ("gate_bias", _p), ("up_scale", _p), ("gate_scale", _p),
                ("glu_op", ctypes.c_int), ("limit", ctypes.c_double)]


def _epilogue(epi: dict | None, keep: list):
    """dict(up_bias=, gate_bias=, up_scale=, gate_scale= (arrays or None),
    glu_op=, limit=) -> ctypes struct (arrays kept alive in keep)."""
    if epi is None:
        return None
    e = _Epilogue()
    for name in ("up_bias", "gate_bias", "up_scale", "gate_scale"):
        v = epi.get(name)
        if v is not None:
            a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
            keep.append(a)
            setattr(e, name, a.ctypes.data)
    e.glu_op = int(epi.get("glu_op", GLU_PLAIN))
    e.limit = float(epi.get("limit", 0.0))
    return ctypes.byref(e), e


def _load(path: str):
    L = ctypes.CDLL(path)
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f16_to_f64.restype = ctypes.c_double
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_quantize_q8_1.argtypes = [_p, _c_i64, _c_i64, _c_i64, _p]
    L.orc_mmvq_rows.argtypes = [_p, ctypes.c_int, _c_i64, _c_i64, _p, _c_i64,
                                _c_i64, _c_i64, _p, _p, _p]
    L.orc_mmvq.argtypes = [_p, ctypes.c_int, _c_i64, _c_i64, _p, _c_i64, _p, _p, _p]
    L.orc_mmvq_glu.argtypes = [_p, _p, ctypes.c_int, _c_i64, _c_i64, _p, _c_i64,
                               ctypes.c_int, _p]
    L.orc_mmvq_id.argtypes = [_p, _c_i64, ctypes.c_int, ctypes.c_int, _c_i64, _c_i64,
                              _p, _c_i64, _p, ctypes.c_int, _p, _p]
    L.orc_mmvq_id_glu.argtypes = [_p, _p, _c_i64, ctypes.c_int, ctypes.c_int, _c_i64,
                                  _c_i64, _p, _c_i64, _p, ctypes.c_int, ctypes.c_int, _p]
    L.orc_glu.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                          ctypes.POINTER(ctypes.c_double)]
    L.orc_mmvq_ex.argtypes = [_p, _p, ctypes.c_int, _c_i64, _c_i64, _p, _c_i64,
                              ctypes.POINTER(_Epilogue), _p]
    L.orc_mmvq_id_ex.argtypes = [_p, _p, _c_i64, ctypes.c_int, ctypes.c_int, _c_i64, _c_i64,
                                 _p, _c_i64, _p, ctypes.c_int, ctypes.POINTER(_Epilogue),
                                 _p, _p, _p, _p]
    L.orc_dequantize_row.argtypes = [ctypes.c_int, _p, _c_i64, _p]
    L.orc_dequantize_q8_1.argtypes = [_p, _c_i64, _p]
    L.orc_q4_k_scale_min.argtypes = [_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int)]
    L.orc_q4_k_scale_min.restype = None
    L.orc_type_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                ctypes.POINTER(ctypes.c_int)]
    L.orc_dots_per_block.argtypes = [ctypes.c_int]
    return L


class Oracle:
    """ctypes wrapper over one build of the oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        self.L = _load(path)

    def f32_to_f16(self, v: float) -> int:
        return int(self.L.orc_f32_to_f16(float(np.float32(v))))

    def f16_to_f64(self, h: int) -> float:
        return float(self.L.orc_f16_to_f64(int(h)))

    def type_info(self, t: int):
        e, b = ctypes.c_int(), ctypes.c_int()
        _check(self.L.orc_type_info(t, ctypes.byref(e), ctypes.byref(b)))
        return e.value, b.value

    def dots_per_block(self, t: int) -> int:
        return int(self.L.orc_dots_per_block(t))

    def q4_k_scale_min(self, scales12, t: int):
        s = _u8(bytes(scales12))
        sc, m = ctypes.c_int(), ctypes.c_int()
        self.L.orc_q4_k_scale_min(_ptr(s), t, ctypes.byref(sc), ctypes.byref(m))
        return sc.value, m.value

    def quantize_q8_1(self, x: np.ndarray, K: int | None = None) -> np.ndarray:
        """x: float32 [n, ldx]; quantizes the first K of each row. Returns uint8
        [n, (K/32)*36]."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x.reshape(1, -1)
        n, ldx = x.shape
        K = ldx if K is None else K
        y = np.zeros((n, (K // 32) * 36), dtype=np.uint8)
        _check(self.L.orc_quantize_q8_1(_ptr(x), K, n, ldx, _ptr(y)))
        return y

    def mmvq(self, W, wtype: int, M: int, K: int, y_q: np.ndarray, n: int,
             rows: tuple[int, int] | None = None, want_dots: bool = False):
        """Returns (out [n, M] f64, mag [n, M] f64, dots or None). With rows=(r0, r1)
        only those rows are filled (others are NaN)."""
        Wb = _u8(W)
        y = _u8(y_q)
        out = np.full((n, M), np.nan)
        mag = np.full((n, M), np.nan)
        dots = None
        dptr = None
        if want_dots:
            qk, _ = BLOCK[wtype]
            dots = np.zeros((n, M, K // qk, DOTS_PER_BLOCK[wtype]), dtype=np.int32)
            dptr = _ptr(dots)
        r0, r1 = rows if rows is not None else (0, M)
        _check(self.L.orc_mmvq_rows(_ptr(Wb), wtype, M, K, _ptr(y), n, r0, r1,
                                   _ptr(out), _ptr(mag), dptr))
        return out, mag, dots

    def mmvq_threaded(self, W, wtype: int, M: int, K: int, y_q: np.ndarray, n: int,
                      threads: int | None = None):
        """All rows, split into contiguous row ranges over host threads (the
        C call releases the interpreter lock). Returns (out [n, M], mag [n, M])."""
        import concurrent.futures as cf
        Wb = _u8(W)
        y = _u8(y_q)
        out = np.full((n, M), np.nan)
        mag = np.full((n, M), np.nan)
        threads = threads or min(16, os.cpu_count() or 1)
        cuts = np.linspace(0, M, min(threads, M) + 1).astype(np.int64)

        def run(i):
            _check(self.L.orc_mmvq_rows(_ptr(Wb), wtype, M, K, _ptr(y), n, int(cuts[i]), int(cuts[i + 1]),
                                       _ptr(out), _ptr(mag), None))

        with cf.ThreadPoolExecutor(max_workers=len(cuts) - 1) as ex:
            list(ex.map(run, range(len(cuts) - 1)))
        return out, mag

    def glu_array(self, glu_op: int, g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
        """orc_glu applied elementwise."""
        gf, uf = np.asarray(g, dtype=np.float64).reshape(-1), np.asarray(u, dtype=np.float64).reshape(-1)
        return np.array([self.glu(glu_op, float(a), float(b), limit) for a, b in zip(gf, uf)]).reshape(
            np.shape(g))

    def mmvq_glu(self, Wg, Wu, wtype: int, M: int, K: int, y_q: np.ndarray, n: int,
                 glu_op: int = GLU_SWIGLU) -> np.ndarray:
        out = np.zeros((n, M))
        _check(self.L.orc_mmvq_glu(_ptr(_u8(Wg)), _ptr(_u8(Wu)), wtype, M, K, _ptr(_u8(y_q)), n,
                                  glu_op, _ptr(out)))
        return out

    def mmvq_id(self, W, expert_stride: int, n_experts: int, wtype: int, M: int, K: int,
                y_q: np.ndarray, n_tokens: int, ids: np.ndarray, top_k: int):
        """Returns (out [n_tokens*top_k, M], mag [n_tokens*top_k, M])."""
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        out = np.zeros((n_tokens * top_k, M))
        mag = np.zeros((n_tokens * top_k, M))
        _check(self.L.orc_mmvq_id(_ptr(_u8(W)), expert_stride, n_experts, wtype, M, K,
                                 _ptr(_u8(y_q)), n_tokens, _ptr(ids), top_k, _ptr(out), _ptr(mag)))
        return out, mag

    def mmvq_id_glu(self, Wg, Wu, expert_stride: int, n_experts: int, wtype: int, M: int, K: int,
                    y_q: np.ndarray, n_tokens: int, ids: np.ndarray, top_k: int,
                    glu_op: int = GLU_SWIGLU) -> np.ndarray:
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        out = np.zeros((n_tokens * top_k, M))
        _check(self.L.orc_mmvq_id_glu(_ptr(_u8(Wg)), _ptr(_u8(Wu)), expert_stride, n_experts,
                                     wtype, M, K, _ptr(_u8(y_q)), n_tokens, _ptr(ids), top_k,
                                     glu_op, _ptr(out)))
        return out

    def glu(self, glu_op: int, g: float, u: float, limit: float = 0.0) -> float:
        out = ctypes.c_double()
        _check(self.L.orc_glu(glu_op, g, u, limit, ctypes.byref(out)))
        return out.value

    def mmvq_ex(self, Wu, Wg, wtype: int, M: int, K: int, y_q: np.ndarray, n: int,
                epi: dict | None = None) -> np.ndarray:
        """Full fused epilogue (Wg None: no gate). Returns out [n, M]."""
        keep: list = []
        ep = _epilogue(epi, keep)
        out = np.zeros((n, M))
        _check(self.L.orc_mmvq_ex(_ptr(_u8(Wu)), None if Wg is None else _ptr(_u8(Wg)), wtype, M, K,
                                 _ptr(_u8(y_q)), n, None if ep is None else ep[0], _ptr(out)))
        return out

    def mmvq_id_ex(self, Wu, Wg, expert_stride: int, n_experts: int, wtype: int, M: int, K: int,
                   y_q: np.ndarray, n_tokens: int, ids: np.ndarray, top_k: int,
                   epi: dict | None = None, shared_up=None, shared_gate=None):
        """Returns (out [n_tokens*top_k, M], shared_out [n_tokens, M] or None)."""
        keep: list = []
        ep = _epilogue(epi, keep)
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        out = np.zeros((n_tokens * top_k, M))
        sh = np.zeros((n_tokens, M)) if shared_up is not None else None
        _check(self.L.orc_mmvq_id_ex(
            _ptr(_u8(Wu)), None if Wg is None else _ptr(_u8(Wg)), expert_stride, n_experts, wtype, M, K,
            _ptr(_u8(y_q)), n_tokens, _ptr(ids), top_k, None if ep is None else ep[0],
            None if shared_up is None else _ptr(_u8(shared_up)),
            None if shared_gate is None else _ptr(_u8(shared_gate)),
            None if sh is None else _ptr(sh), _ptr(out)))
        return out, sh

    def dequantize_row(self, wtype: int, row, K: int) -> np.ndarray:
        w = np.zeros(K)
        _check(self.L.orc_dequantize_row(wtype, _ptr(_u8(row)), K, _ptr(w)))
        return w

    def dequantize_q8_1(self, y_col, K: int) -> np.ndarray:
        y = np.zeros(K)
        _check(self.L.orc_dequantize_q8_1(_ptr(_u8(y_col)), K, _ptr(y)))
        return y


_default = None


def default() -> Oracle:
    """The oracle built from oracle/mmvq_oracle.c (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build(force=False)
        _default = Oracle(LIB)
    return _default
