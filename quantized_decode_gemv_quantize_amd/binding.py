"""Python binding of ``libmmvq.so`` (C ABI in ``include/mmvq.h``).

Argument marshalling only: every step of the computation runs in the HIP
library. Functions keep the C names; device buffers may be given as torch
tensors (their ``data_ptr()`` is passed) or as raw integer addresses, and
``stream`` as a torch stream, a raw ``hipStream_t`` integer, or ``None`` for
torch's current stream. A non-zero return code raises ``MMVQError``.

There is no fallback: if the library has not been built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmmvq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mmvq.h")

Q4_0, Q8_0, Q8_1, Q4_K, Q6_K = 2, 8, 9, 12, 14
Q4_1, Q5_0, Q5_1, Q5_K = 3, 6, 7, 13
GLU_PLAIN, GLU_SWIGLU, GLU_GEGLU, GLU_SWIGLU_OAI, GLU_SWIGLU_CLAMP = 0, 1, 2, 3, 4
MAX_COLS = 8
BLOCK = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210), Q8_1: (32, 36)}
DOTS_PER_BLOCK = {Q4_0: 1, Q8_0: 1, Q4_K: 16, Q6_K: 16}

ERR_NULL, ERR_TYPE, ERR_SHAPE, ERR_ALIGN, ERR_LAUNCH = -1, -2, -3, -4, -5

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p

class Epilogue(ctypes.Structure):
    """``mmvq_epilogue``: device pointers (ints, tensors via ``epilogue()``)."""
    _fields_ = [("up_bias", _p), ("gate_bias", _p), ("up_scale", _p), ("gate_scale", _p),
                ("glu_op", _int), ("glu_limit", ctypes.c_float)]


def epilogue(up_bias=None, gate_bias=None, up_scale=None, gate_scale=None, glu_op: int = 0,
             glu_limit: float = 0.0) -> Epilogue:
    e = Epilogue()
    e.up_bias, e.gate_bias = _addr(up_bias), _addr(gate_bias)
    e.up_scale, e.gate_scale = _addr(up_scale), _addr(gate_scale)
    e.glu_op, e.glu_limit = glu_op, glu_limit
    return e


_EP = ctypes.POINTER(Epilogue)

_SIGS = {
    "mmvq_type_info": (_int, [_int, ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "mmvq_many_columns_min": (_int, [_int, _int, _int, ctypes.POINTER(_int)]),
    "mmvq_quantize_q8_1": (_int, [_p, _i64, _i64, _i64, _p, _p]),
    "mmvq": (_int, [_p, _int, _i64, _i64, _p, _i64, _p, _p]),
    "mmvq_glu": (_int, [_p, _p, _int, _i64, _i64, _p, _i64, _int, _p, _p]),
    "mmvq_id": (_int, [_p, _i64, _int, _int, _i64, _i64, _p, _i64, _p, _int, _p, _p]),
    "mmvq_id_glu": (_int, [_p, _p, _i64, _int, _int, _i64, _i64, _p, _i64, _p, _int, _int, _p, _p]),
    "mmvq_f32": (_int, [_p, _int, _i64, _i64, _p, _i64, _i64, _p, _p]),
    "mmvq_glu_f32": (_int, [_p, _p, _int, _i64, _i64, _p, _i64, _i64, _int, _p, _p]),
    "mmvq_id_f32": (_int, [_p, _i64, _int, _int, _i64, _i64, _p, _i64, _i64, _p, _int, _p, _p]),
    "mmvq_id_glu_f32": (_int, [_p, _p, _i64, _int, _int, _i64, _i64, _p, _i64, _i64, _p, _int, _int,
                               _p, _p]),
    "mmvq_ex": (_int, [_p, _p, _int, _i64, _i64, _p, _p, _i64, _i64, _EP, _p, _p]),
    "mmvq_id_ex": (_int, [_p, _p, _i64, _int, _int, _i64, _i64, _p, _p, _i64, _i64, _p, _int, _EP,
                          _p, _p, _p, _p, _p]),
    "mmvq_block_dots": (_int, [_p, _int, _i64, _i64, _p, _i64, _p, _p]),
    "mmvq_read_probe": (_int, [_p, _i64, _p, _p]),
    "mmvq_strerror": (ctypes.c_char_p, [_int]),
}

_lib = None


class MMVQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code}: {mmvq_strerror(code)}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with "
                               "`python -m quantized_decode_gemv_quantize_amd.build`")
        L = ctypes.CDLL(LIB)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_symbols(header: str = HEADER) -> list[str]:
    """Function names declared in include/mmvq.h."""
    text = open(header).read()
    return re.findall(r"^\s*(?:int|const char \*)\s*(mmvq\w*)\s*\(", text, flags=re.M)


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, rc: int) -> int:
    if rc != 0:
        raise MMVQError(fn, rc)
    return rc


def mmvq_strerror(code: int) -> str:
    return lib().mmvq_strerror(code).decode()


def mmvq_type_info(wtype: int) -> tuple[int, int]:
    e, b = _int(), _int()
    _check("mmvq_type_info", lib().mmvq_type_info(wtype, ctypes.byref(e), ctypes.byref(b)))
    return e.value, b.value


def mmvq_many_columns_min(wtype: int, gated: bool, fp32: bool = False) -> int:
    n = _int()
    _check("mmvq_many_columns_min",
           lib().mmvq_many_columns_min(wtype, int(bool(gated)), int(bool(fp32)), ctypes.byref(n)))
    return n.value


def mmvq_quantize_q8_1(x, K: int, n: int, ldx: int, y_q, stream=None) -> None:
    _check("mmvq_quantize_q8_1",
           lib().mmvq_quantize_q8_1(_addr(x), K, n, ldx, _addr(y_q), _stream(stream)))


def mmvq(W, wtype: int, M: int, K: int, y_q, n: int, out, stream=None) -> None:
    _check("mmvq", lib().mmvq(_addr(W), wtype, M, K, _addr(y_q), n, _addr(out), _stream(stream)))


def mmvq_glu(W_gate, W_up, wtype: int, M: int, K: int, y_q, n: int, glu_op: int, out,
             stream=None) -> None:
    _check("mmvq_glu", lib().mmvq_glu(_addr(W_gate), _addr(W_up), wtype, M, K, _addr(y_q), n,
                                      glu_op, _addr(out), _stream(stream)))


def mmvq_id(W, expert_stride_bytes: int, n_experts: int, wtype: int, M: int, K: int, y_q,
            n_tokens: int, ids, top_k: int, out, stream=None) -> None:
    _check("mmvq_id", lib().mmvq_id(_addr(W), expert_stride_bytes, n_experts, wtype, M, K,
                                    _addr(y_q), n_tokens, _addr(ids), top_k, _addr(out),
                                    _stream(stream)))


def mmvq_id_glu(W_gate, W_up, expert_stride_bytes: int, n_experts: int, wtype: int, M: int,
                K: int, y_q, n_tokens: int, ids, top_k: int, glu_op: int, out,
                stream=None) -> None:
    _check("mmvq_id_glu", lib().mmvq_id_glu(_addr(W_gate), _addr(W_up), expert_stride_bytes,
                                            n_experts, wtype, M, K, _addr(y_q), n_tokens,
                                            _addr(ids), top_k, glu_op, _addr(out),
                                            _stream(stream)))


def mmvq_f32(W, wtype: int, M: int, K: int, x, n: int, ldx: int, out, stream=None) -> None:
    _check("mmvq_f32", lib().mmvq_f32(_addr(W), wtype, M, K, _addr(x), n, ldx, _addr(out),
                                      _stream(stream)))


def mmvq_glu_f32(W_gate, W_up, wtype: int, M: int, K: int, x, n: int, ldx: int, glu_op: int,
                 out, stream=None) -> None:
    _check("mmvq_glu_f32", lib().mmvq_glu_f32(_addr(W_gate), _addr(W_up), wtype, M, K, _addr(x),
                                              n, ldx, glu_op, _addr(out), _stream(stream)))


def mmvq_id_f32(W, expert_stride_bytes: int, n_experts: int, wtype: int, M: int, K: int, x,
                n_tokens: int, ldx: int, ids, top_k: int, out, stream=None) -> None:
    _check("mmvq_id_f32", lib().mmvq_id_f32(_addr(W), expert_stride_bytes, n_experts, wtype, M, K,
                                            _addr(x), n_tokens, ldx, _addr(ids), top_k,
                                            _addr(out), _stream(stream)))


def mmvq_id_glu_f32(W_gate, W_up, expert_stride_bytes: int, n_experts: int, wtype: int, M: int,
                    K: int, x, n_tokens: int, ldx: int, ids, top_k: int, glu_op: int, out,
                    stream=None) -> None:
    _check("mmvq_id_glu_f32", lib().mmvq_id_glu_f32(_addr(W_gate), _addr(W_up),
                                                    expert_stride_bytes, n_experts, wtype, M, K,
                                                    _addr(x), n_tokens, ldx, _addr(ids), top_k,
                                                    glu_op, _addr(out), _stream(stream)))


def _ep(epi):
    return None if epi is None else ctypes.byref(epi)


def mmvq_ex(W_up, W_gate, wtype: int, M: int, K: int, y_q, x, ldx: int, n: int,
            epi: Epilogue | None, out, stream=None) -> None:
    _check("mmvq_ex", lib().mmvq_ex(_addr(W_up), _addr(W_gate), wtype, M, K, _addr(y_q), _addr(x), ldx,
                                    n, _ep(epi), _addr(out), _stream(stream)))


def mmvq_id_ex(W_up, W_gate, expert_stride_bytes: int, n_experts: int, wtype: int, M: int, K: int,
               y_q, x, ldx: int, n_tokens: int, ids, top_k: int, epi: Epilogue | None,
               shared_up, shared_gate, shared_out, out, stream=None) -> None:
    _check("mmvq_id_ex", lib().mmvq_id_ex(_addr(W_up), _addr(W_gate), expert_stride_bytes, n_experts,
                                          wtype, M, K, _addr(y_q), _addr(x), ldx, n_tokens, _addr(ids),
                                          top_k, _ep(epi), _addr(shared_up), _addr(shared_gate),
                                          _addr(shared_out), _addr(out), _stream(stream)))


def mmvq_block_dots(W, wtype: int, M: int, K: int, y_q, n: int, dots, stream=None) -> None:
    _check("mmvq_block_dots", lib().mmvq_block_dots(_addr(W), wtype, M, K, _addr(y_q), n,
                                                    _addr(dots), _stream(stream)))


# ---------------------------------------------------------------------------
# Tensor-level conveniences (allocate outputs with torch, then call the ABI)
# ---------------------------------------------------------------------------

def mmvq_read_probe(src, nbytes: int, sink, stream=None) -> None:
    _check("mmvq_read_probe", lib().mmvq_read_probe(_addr(src), nbytes, _addr(sink), _stream(stream)))


def quantize(x, K: int | None = None, stream=None):
    """x: float32 CUDA tensor [n, ldx] -> uint8 tensor [n, (K/32)*36]."""
    import torch
    if x.dim() == 1:
        x = x.view(1, -1)
    n, ldx = x.shape
    K = ldx if K is None else K
    y = torch.empty((n, K // 32 * 36), dtype=torch.uint8, device=x.device)
    mmvq_quantize_q8_1(x, K, n, x.stride(0), y, stream)
    return y


def gemv(W, wtype: int, M: int, K: int, y_q, n: int, stream=None):
    """-> float32 tensor [n, M]."""
    import torch
    out = torch.empty((n, M), dtype=torch.float32, device=y_q.device)
    mmvq(W, wtype, M, K, y_q, n, out, stream)
    return out
