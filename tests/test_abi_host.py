"""The C-ABI library without a GPU: it loads, exports every function that
include/mmvq.h declares, reports the block geometry, and rejects invalid
arguments with the documented codes before touching any device (argument
checks run on the host and enqueue nothing)."""
import ctypes

import pytest

from quantized_decode_gemv_quantize_amd import binding as B


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = B.declared_symbols()
    assert set(names) == {"mmvq_type_info", "mmvq_quantize_q8_1", "mmvq", "mmvq_glu", "mmvq_id",
                          "mmvq_id_glu", "mmvq_f32", "mmvq_glu_f32", "mmvq_id_f32", "mmvq_id_glu_f32",
                          "mmvq_ex", "mmvq_id_ex", "mmvq_block_dots", "mmvq_read_probe", "mmvq_strerror",
                          "mmvq_many_columns_min"}
    for n in names:
        assert hasattr(L, n), n


def test_type_info():
    assert B.mmvq_type_info(B.Q4_0) == (32, 18)
    assert B.mmvq_type_info(B.Q8_0) == (32, 34)
    assert B.mmvq_type_info(B.Q4_K) == (256, 144)
    assert B.mmvq_type_info(B.Q6_K) == (256, 210)
    assert B.mmvq_type_info(B.Q8_1) == (32, 36)
    assert B.mmvq_type_info(B.Q4_1) == (32, 20)
    assert B.mmvq_type_info(B.Q5_0) == (32, 22)
    assert B.mmvq_type_info(B.Q5_1) == (32, 24)
    assert B.mmvq_type_info(B.Q5_K) == (256, 176)
    with pytest.raises(B.MMVQError) as e:
        B.mmvq_type_info(5)
    assert e.value.code == B.ERR_TYPE
    assert B.lib().mmvq_type_info(B.Q4_K, None, None) == 0


def test_many_columns_min(L):
    """The documented crossover table, and its errors."""
    plain = {B.Q5_K: 5, B.Q4_K: 6, B.Q6_K: 7, B.Q4_0: 8, B.Q5_0: 8, B.Q8_0: 8, B.Q4_1: 9, B.Q5_1: 9}
    gated = {B.Q5_K: 5, B.Q4_K: 7, B.Q6_K: 9, B.Q4_0: 9, B.Q5_0: 9, B.Q8_0: 9, B.Q4_1: 9, B.Q5_1: 9}
    plain_f32 = {B.Q5_K: 8, B.Q4_K: 9, B.Q6_K: 6, B.Q4_0: 9, B.Q5_0: 9, B.Q8_0: 9, B.Q4_1: 9, B.Q5_1: 9}
    gated_f32 = {B.Q5_K: 4, B.Q4_K: 5, B.Q6_K: 5, B.Q4_0: 4, B.Q5_0: 4, B.Q8_0: 5, B.Q4_1: 5, B.Q5_1: 5}
    for t in plain:
        assert B.mmvq_many_columns_min(t, False) == plain[t]
        assert B.mmvq_many_columns_min(t, True) == gated[t]
        assert B.mmvq_many_columns_min(t, False, fp32=True) == plain_f32[t]
        assert B.mmvq_many_columns_min(t, True, fp32=True) == gated_f32[t]
    for t in (5, B.Q8_1, -1):
        for f in (False, True):
            with pytest.raises(B.MMVQError) as e:
                B.mmvq_many_columns_min(t, False, fp32=f)
            assert e.value.code == B.ERR_TYPE
    assert L.mmvq_many_columns_min(B.Q4_K, 0, 0, None) == B.ERR_NULL
    assert L.mmvq_many_columns_min(B.Q4_K, 1, 1, None) == B.ERR_NULL


def test_strerror(L):
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(B.mmvq_strerror(code), str) and B.mmvq_strerror(code)


# Fake, never dereferenced addresses: validation fails before any device work.
P16, P4 = 1 << 20, (1 << 20) + 4


@pytest.mark.parametrize("args,code", [
    ((None, B.Q4_K, 1, 256, P16, 1, P16), B.ERR_NULL),
    ((P16, B.Q4_K, 1, 256, None, 1, P16), B.ERR_NULL),
    ((P16, B.Q4_K, 1, 256, P16, 1, None), B.ERR_NULL),
    ((P16, 5, 1, 256, P16, 1, P16), B.ERR_TYPE),
    ((P16, B.Q8_1, 1, 256, P16, 1, P16), B.ERR_TYPE),
    ((P16, B.Q4_K, 1, 200, P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q4_0, 1, 48, P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q8_0, 1, 48, P16, 1, P16), B.ERR_SHAPE),
    # rows of more than 2^24 units (longer rows are walked in chunks)
    ((P16, B.Q8_0, 1, 32 * ((1 << 24) + 1), P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q4_0, 1, 32 * ((1 << 24) + 1), P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q4_K, 0, 256, P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q4_K, 1, 256, P16, 0, P16), B.ERR_SHAPE),
    ((P16, B.Q4_K, 1, 256, P16, 257, P16), B.ERR_SHAPE),
    ((P16, B.Q4_0, 1, 256, P16, 257, P16), B.ERR_SHAPE),
    ((P16, B.Q6_K, 1, 256, P16, 257, P16), B.ERR_SHAPE),
    ((P16, B.Q4_0, 1, 96, P16, 257, P16), B.ERR_SHAPE),
    ((P16, B.Q4_K, 1, 256 * ((1 << 22) + 1), P16, 1, P16), B.ERR_SHAPE),
    ((P16, B.Q6_K, 1, 256 * ((1 << 22) + 1), P16, 1, P16), B.ERR_SHAPE),
    # M * K above 2^40
    ((P16, B.Q4_K, 1 << 20, 256 * 4097, P16, 1, P16), B.ERR_SHAPE),
    ((P4, B.Q4_K, 1, 256, P16, 1, P16), B.ERR_ALIGN),
    ((P16, B.Q4_K, 1, 256, P4, 1, P16), B.ERR_ALIGN),
    ((P16, B.Q4_K, 1, 256, P16, 1, P16 + 2), B.ERR_ALIGN),
])
def test_mmvq_argument_checks(L, args, code):
    assert L.mmvq(*args, None) == code


def test_other_entry_points_argument_checks(L):
    assert L.mmvq_glu(None, P16, B.Q4_K, 1, 256, P16, 1, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_glu(P16, P16, B.Q4_K, 1, 256, P16, 1, 7, P16, None) == B.ERR_TYPE
    # the clamp op needs a limit, which only the epilogue form carries
    assert L.mmvq_glu(P16, P16, B.Q4_K, 1, 256, P16, 1, B.GLU_SWIGLU_CLAMP, P16, None) == B.ERR_TYPE
    assert L.mmvq_glu_f32(P16, P16, B.Q4_K, 1, 256, P16, 1, 256, B.GLU_SWIGLU_CLAMP, P16, None) == B.ERR_TYPE
    assert L.mmvq_read_probe(None, 64, P16, None) == B.ERR_NULL
    assert L.mmvq_read_probe(P16, 0, P16, None) == B.ERR_SHAPE
    assert L.mmvq_read_probe(P16, 24, P16, None) == B.ERR_SHAPE
    assert L.mmvq_read_probe(P4, 64, P16, None) == B.ERR_ALIGN
    assert L.mmvq_glu(P4, P16, B.Q4_K, 1, 256, P16, 1, 1, P16, None) == B.ERR_ALIGN
    assert L.mmvq_id(P16, 288, 4, B.Q4_K, 2, 256, P16, 1, None, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_id(P16, 144, 4, B.Q4_K, 2, 256, P16, 1, P16, 1, P16, None) == B.ERR_SHAPE
    assert L.mmvq_id(P16, 288, 4, B.Q4_K, 2, 256, P16, 1, P16, 5, P16, None) == B.ERR_SHAPE
    assert L.mmvq_id(P16, 288, 4, B.Q4_K, 2, 256, P16, 9, P16, 1, P16, None) == B.ERR_SHAPE
    assert L.mmvq_id(P16, 296, 4, B.Q4_K, 2, 256, P16, 1, P16, 1, P16, None) == B.ERR_ALIGN
    assert L.mmvq_id(P16, 288, 0, B.Q4_K, 2, 256, P16, 1, P16, 1, P16, None) == B.ERR_SHAPE
    assert L.mmvq_id_glu(None, P16, 288, 4, B.Q4_K, 2, 256, P16, 1, P16, 1, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_id_glu(P16, P16, 288, 4, B.Q4_K, 2, 256, P16, 1, P16, 1, 9, P16, None) == B.ERR_TYPE
    assert L.mmvq_block_dots(P16, B.Q4_K, 1, 100, P16, 1, P16, None) == B.ERR_SHAPE
    assert L.mmvq_quantize_q8_1(None, 32, 1, 32, P16, None) == B.ERR_NULL
    assert L.mmvq_quantize_q8_1(P16, 33, 1, 33, P16, None) == B.ERR_SHAPE
    assert L.mmvq_quantize_q8_1(P16, 32, 1, 16, P16, None) == B.ERR_SHAPE
    assert L.mmvq_quantize_q8_1(P16, 32, 257, 32, P16, None) == B.ERR_SHAPE
    assert L.mmvq_quantize_q8_1(P16 + 2, 32, 1, 32, P16, None) == B.ERR_ALIGN
    assert L.mmvq_quantize_q8_1(P16, 32, 1, 32, P4, None) == B.ERR_ALIGN


def test_f32_entry_points_argument_checks(L):
    assert L.mmvq_f32(P16, B.Q4_K, 1, 256, None, 1, 256, P16, None) == B.ERR_NULL
    assert L.mmvq_f32(None, B.Q4_K, 1, 256, P16, 1, 256, P16, None) == B.ERR_NULL
    assert L.mmvq_f32(P16, B.Q8_1, 1, 256, P16, 1, 256, P16, None) == B.ERR_TYPE
    assert L.mmvq_f32(P16, B.Q4_K, 1, 256, P16, 1, 255, P16, None) == B.ERR_SHAPE
    assert L.mmvq_f32(P16, B.Q4_K, 1, 256, P16, 257, 256, P16, None) == B.ERR_SHAPE
    K = 256 * ((1 << 22) + 1)
    assert L.mmvq_f32(P16, B.Q4_K, 1, K, P16, 1, K, P16, None) == B.ERR_SHAPE
    assert L.mmvq_f32(P16, B.Q4_K, 1, 256, P16 + 2, 1, 256, P16, None) == B.ERR_ALIGN
    # fp32 x needs only 4-byte alignment (q8_1 columns need 16)
    assert L.mmvq_f32(P4, B.Q4_K, 1, 256, P16, 1, 256, P16, None) == B.ERR_ALIGN
    assert L.mmvq_glu_f32(None, P16, B.Q4_K, 1, 256, P16, 1, 256, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_glu_f32(P16, P16, B.Q4_K, 1, 256, P16, 1, 256, 5, P16, None) == B.ERR_TYPE
    assert L.mmvq_glu_f32(P16, P16, B.Q4_K, 1, 256, None, 1, 256, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_id_f32(P16, 288, 4, B.Q4_K, 2, 256, P16, 1, 256, None, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_id_f32(P16, 288, 4, B.Q4_K, 2, 256, P16, 1, 100, P16, 1, P16, None) == B.ERR_SHAPE
    assert L.mmvq_id_f32(P16, 288, 4, B.Q4_K, 2, 256, None, 1, 256, P16, 1, P16, None) == B.ERR_NULL
    assert L.mmvq_id_glu_f32(P16, P16, 288, 4, B.Q4_K, 2, 256, P16, 1, 256, P16, 1, 9, P16,
                             None) == B.ERR_TYPE
    assert L.mmvq_id_glu_f32(P16, P16, 288, 4, B.Q4_K, 2, 256, P16, 1, 256, P16, 5, 1, P16,
                             None) == B.ERR_SHAPE


def test_ex_entry_points_argument_checks(L):
    e = B.epilogue(glu_op=B.GLU_SWIGLU)
    bad_op = B.epilogue(glu_op=5)
    bad_bias = B.epilogue(up_bias=P16 + 2)
    ref = ctypes.byref
    # activation operand: neither -> NULL, both -> SHAPE
    assert L.mmvq_ex(P16, None, B.Q4_K, 1, 256, None, None, 0, 1, ref(e), P16, None) == B.ERR_NULL
    assert L.mmvq_ex(P16, None, B.Q4_K, 1, 256, P16, P16, 256, 1, ref(e), P16, None) == B.ERR_SHAPE
    assert L.mmvq_ex(P16, P16, B.Q4_K, 1, 256, P16, None, 0, 1, ref(bad_op), P16, None) == B.ERR_TYPE
    assert L.mmvq_ex(P16, None, B.Q4_K, 1, 256, P16, None, 0, 1, ref(bad_bias), P16, None) == B.ERR_ALIGN
    assert L.mmvq_ex(P16, P4, B.Q4_K, 1, 256, P16, None, 0, 1, ref(e), P16, None) == B.ERR_ALIGN
    assert L.mmvq_ex(P16, None, B.Q4_K, 1, 256, None, P16, 255, 1, None, P16, None) == B.ERR_SHAPE
    args = (P16, 288, 4, B.Q4_K, 2, 256, P16, None, 0, 1, P16, 1, ref(e))
    # shared expert: output required; a gate form needs the shared gate too
    assert L.mmvq_id_ex(P16, None, *args[1:], P16, None, None, P16, None) == B.ERR_NULL
    assert L.mmvq_id_ex(P16, P16, *args[1:], P16, None, P16, P16, None) == B.ERR_NULL
    assert L.mmvq_id_ex(P16, P16, *args[1:], P4, P16, P16, P16, None) == B.ERR_ALIGN
    assert L.mmvq_id_ex(P16, None, 288, 65535, B.Q4_K, 2, 256, P16, None, 0, 1, P16, 1, ref(e),
                        P16, None, P16, P16, None) == B.ERR_SHAPE


def test_binding_raises_with_code():
    with pytest.raises(B.MMVQError) as e:
        B.mmvq(P16, B.Q4_K, 1, 200, P16, 1, P16, stream=0)
    assert e.value.code == B.ERR_SHAPE and "invalid shape" in str(e.value)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB", str(tmp_path / "absent.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
    assert ctypes  # keep import used
