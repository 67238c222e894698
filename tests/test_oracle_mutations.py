"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/mmvq_oracle.c`` to a temporary directory, applies
one textual change that models a plausible mistake (a dropped term, a wrong
sign, index or shift, a swapped operand, another rounding rule), builds it
with gcc and runs the pin suite on it. At least one pin must fail. The
oracle in the repository is never modified.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "q8_1_ties_to_even": ("(int)roundf(xb[i] / d)", "(int)rintf(xb[i] / d)"),
    "q8_1_s_without_d": ("const float s = d * (float)sumq;", "const float s = (float)sumq;"),
    "q8_1_divides_by_fp16_d": ("(int)roundf(xb[i] / d)",
                               "(int)roundf(xb[i] / (float)orc_f16_to_f64(orc_f32_to_f16(d)))"),
    "q8_1_scale_128": ("const float d = amax / 127.0f;", "const float d = amax / 128.0f;"),
    "f16_ties_up": ("return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;", "return fl + 1.0;"),
    "q4_0_nibbles_swapped": ("const uint8_t *qs = blk + 2;\n    return e < 16 ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);",
                             "const uint8_t *qs = blk + 2;\n    return e < 16 ? (qs[e] >> 4) : (qs[e - 16] & 0x0F);"),
    "q4_0_zero_point_7": ("const double t2 = 8.0 * dw * q8_s(ycol, qb);",
                          "const double t2 = 7.0 * dw * q8_s(ycol, qb);"),
    "q4_0_no_zero_point": ("const double t2 = 8.0 * dw * q8_s(ycol, qb);",
                           "const double t2 = 0.0 * dw * q8_s(ycol, qb);"),
    "k_min_magnitude_whole_sub_blocks": (
        "for (int h = 0; h < 2; ++h) *mag += fabs(d * sc * d8 * half1[h]) + fabs(dmin * m * d8 * half2[h]);",
        "*mag += fabs(t1) + fabs(t2);"),
    "q4_k_min_sign": ("const double t2 = dmin * m * d8 * dot2;\n        *acc += t1 - t2;",
                      "const double t2 = dmin * m * d8 * dot2;\n        *acc += t1 + t2;"),
    "q4_k_d_dmin_swapped": ("const double dmin = orc_f16_to_f64(rd16(blk + 2));",
                            "const double dmin = orc_f16_to_f64(rd16(blk));"),
    "q4_k_scale_high_bits_from_t": ("*sc = (B[t + 4] & 15) | ((B[t - 4] >> 6) << 4);",
                                    "*sc = (B[t + 4] & 15) | ((B[t] >> 6) << 4);"),
    "q4_k_min_low_bits_from_scale_byte": ("*m = B[t + 4] & 63;", "*m = B[t] & 63;"),
    "q4_k_nibble_parity_swapped": ("return (t % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                                   "return (t % 2 == 1) ? (byte & 0x0F) : (byte >> 4);"),
    "q4_k_chunk_index": ("blk + 16;\n    const int t = e / 32, l = e % 32, c = t / 2;\n    const uint8_t byte = qs[32 * c + l];",
                         "blk + 16;\n    const int t = e / 32, l = e % 32, c = t / 2;\n    const uint8_t byte = qs[32 * (t % 4) + l];"),
    "q4_k_wrong_q8_block": ("const int qy = q8_q(ycol, qb + t, l);",
                            "const int qy = q8_q(ycol, qb + (t ^ 1), l);"),
    "q4_k_field_order": ("const uint8_t *qs = blk + 16;\n    const int t = e / 32",
                         "const uint8_t *qs = blk + 0;\n    const int t = e / 32"),
    "q6_k_high_shift": ("const int high = (qh[32 * h + l] >> (2 * g)) & 3;",
                        "const int high = (qh[32 * h + l] >> g) & 3;"),
    "q6_k_low_half_select": ("ql[64 * h + 32 * (g % 2) + l]", "ql[64 * h + 32 * (g / 2) + l]"),
    "q6_k_offset_31": ("isum += (q6_k_code(blk, e) - 32)", "isum += (q6_k_code(blk, e) - 31)"),
    "q6_k_q8_block_map": ("const int64_t yb = qb + s / 2;", "const int64_t yb = qb + s % 8;"),
    "q6_k_scale_unsigned": ("return (int8_t)blk[192 + s];", "return blk[192 + s];"),
    "legacy_nibbles_swapped": ("static int nib_code(const uint8_t *qs, int e) { return e < 16 ? (qs[e] & 0x0F) : (qs[e - 16] >> 4); }",
                               "static int nib_code(const uint8_t *qs, int e) { return e < 16 ? (qs[e] >> 4) : (qs[e - 16] & 0x0F); }"),
    "qh_bit_big_endian": ("return (qh[e / 8] >> (e % 8)) & 1;", "return (qh[3 - e / 8] >> (e % 8)) & 1;"),
    "q4_1_field_order": ("static int q4_1_code(const uint8_t *blk, int e) { return nib_code(blk + 4, e); }",
                         "static int q4_1_code(const uint8_t *blk, int e) { return nib_code(blk + 2, e); }"),
    "q5_1_qh_after_qs": ("static int q5_1_code(const uint8_t *blk, int e) { return nib_code(blk + 8, e) | (qh_bit(blk + 4, e) << 4); }",
                         "static int q5_1_code(const uint8_t *blk, int e) { return nib_code(blk + 4, e) | (qh_bit(blk + 20, e) << 4); }"),
    "q5_0_zero_point_8": ("const double t2 = type == ORC_Q5_0 ? -16.0 * d * q8_s(ycol, qb)",
                          "const double t2 = type == ORC_Q5_0 ? -8.0 * d * q8_s(ycol, qb)"),
    "legacy_offset_sign": ("*acc += t1 + t2;", "*acc += t1 - t2;"),
    "q5_k_qh_bit_chunk": ("return low | (((qh[l] >> t) & 1) << 4);", "return low | (((qh[l] >> c) & 1) << 4);"),
    "q5_k_qs_offset": ("const uint8_t *qh = blk + 16, *qs = blk + 48;", "const uint8_t *qh = blk + 16, *qs = blk + 16;"),
    "silu_sigmoid_only": ("static double silu(double z) { return z / (1.0 + exp(-z)); }",
                          "static double silu(double z) { return 1.0 / (1.0 + exp(-z)); }"),
    "glu_plain_for_silu": ("case ORC_GLU_SWIGLU: *out = silu(g) * u; break;",
                           "case ORC_GLU_SWIGLU: *out = g * u; break;"),
    "id_slot_as_token": ("rc = orc_mmvq(We, type, M, K, y_q + t * (K / 32) * 36, 1,",
                         "rc = orc_mmvq(We, type, M, K, y_q + k * (K / 32) * 36, 1,"),
    "gelu_cubic_dropped": ("tanh(c * (z + 0.044715 * z * z * z))", "tanh(c * z)"),
    "gelu_erf_form": ("return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));",
                      "(void)c; return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));"),
    "oai_no_plus_one": ("* (uc + 1.0);\n        break;", "* uc;\n        break;"),
    "oai_alpha_dropped": ("exp(-ORC_OAI_ALPHA * gc)", "exp(-gc)"),
    "oai_limit_from_caller": ("const double gc = g < ORC_OAI_LIMIT ? g : ORC_OAI_LIMIT;",
                              "const double gc = g < limit ? g : limit;"),
    "clamp_up_one_sided": ("const double uc = u < -limit ? -limit : (u > limit ? limit : u);",
                           "const double uc = u > limit ? limit : u;"),
    "clamp_gate_both_sides": ("const double gc = g < limit ? g : limit;",
                              "const double gc = g < -limit ? -limit : (g < limit ? g : limit);"),
    "epilogue_bias_before_scale": ("if (epi->up_scale) u *= epi->up_scale[e];\n    if (epi->up_bias) u += epi->up_bias[(int64_t)e * M + r];",
                                   "if (epi->up_bias) u += epi->up_bias[(int64_t)e * M + r];\n    if (epi->up_scale) u *= epi->up_scale[e];"),
    "epilogue_gate_bias_from_up": ("g += epi->gate_bias[", "g += epi->up_bias["),
    "id_ex_bias_of_expert_0": ("if (epi->up_bias) u += epi->up_bias[(int64_t)e * M + r];",
                               "if (epi->up_bias) u += epi->up_bias[r];"),
    "shared_expert_gate_up_swapped": ("rc = orc_glu(epi ? epi->glu_op : ORC_GLU_PLAIN, g, u,",
                                      "rc = orc_glu(epi ? epi->glu_op : ORC_GLU_PLAIN, u, g,"),
    "q8_0_unsigned_codes": ("static int q8_0_code(const uint8_t *blk, int e) { return (int8_t)blk[2 + e]; }",
                            "static int q8_0_code(const uint8_t *blk, int e) { return blk[2 + e]; }"),
    "q8_0_codes_at_0": ("return (int8_t)blk[2 + e]; }", "return (int8_t)blk[e]; }"),
    "q8_0_zero_point": ("isum += q8_0_code(blk, e) * q8_q(ycol, qb, e);",
                        "isum += (q8_0_code(blk, e) - 1) * q8_q(ycol, qb, e);"),
    "columns_share_first": ("row_dot(W + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &acc, &mg,",
                            "row_dot(W + r * nb * bb, type, nb, bb, qk, y_q, &acc, &mg,"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, source, name):
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mmvq_oracle.c"
    src.write_text(source.replace(old, new))
    hdr = os.path.join(oracle.HERE, "mmvq_oracle.h")
    (tmp_path / "mmvq_oracle.h").write_text(open(hdr).read())
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(lib), str(src), "-lm"])
    mutant = oracle.Oracle(str(lib))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"planted mistake {name} passed every pin"
