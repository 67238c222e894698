/*
 * mmvq_oracle.c - plain CPU oracle for the decode-time quantized mat-vec.
 *
 * TEST INFRASTRUCTURE ONLY (see mmvq_oracle.h): loaded by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product.
 *
 * Style: scalar loops over elements, fp64 accumulation, one helper per
 * block format that returns the code of one element. Nothing is blocked,
 * fused or reordered beyond what the definitions state. Build with
 * -ffp-contract=off and without -ffast-math: the q8_1 step is defined in
 * fp32 and must round exactly as written.
 *
 * Parity pins live in tests/test_oracle_*.py; the readings taken where the
 * pages are silent are listed next to the code that takes them.
 */
#include "mmvq_oracle.h"

#include <math.h>
#include <stddef.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16                                                        */
/* ------------------------------------------------------------------------ */

double orc_f16_to_f64(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24   */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);   /* (1024+f) * 2^(e-15-10) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to even. The
 * callers pass exact values (a float scaled by a power of two). */
static double round_half_even(double q) {
    const double fl = floor(q);
    const double diff = q - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

uint16_t orc_f32_to_f16(float f) {
    const double x = (double)f;          /* exact */
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);   /* rounds to inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; m == 1024 is the smallest normal */
        const double m = round_half_even(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int ex;
    (void)frexp(a, &ex);                 /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;                      /* a in [2^E, 2^(E+1))           */
    double m = round_half_even(a / ldexp(1.0, E - 10));   /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

/* ------------------------------------------------------------------------ */
/* Type table [GGUF16 §16.1.2, §16.1.3]; [MMVQ §权重的排法, §激活的量化]     */
/* ------------------------------------------------------------------------ */

int orc_type_info(int type, int *block_elems, int *block_bytes) {
    int e, b;
    switch (type) {
    case ORC_Q4_0: e = 32;  b = 18;  break;   /* half d + 16 bytes of nibbles      */
    case ORC_Q4_1: e = 32;  b = 20;  break;   /* half d, half m + 16 bytes          */
    case ORC_Q5_0: e = 32;  b = 22;  break;   /* half d, 4 bytes of 5th bits, 16    */
    case ORC_Q5_1: e = 32;  b = 24;  break;   /* half d, half m, 4 + 16 bytes       */
    case ORC_Q8_0: e = 32;  b = 34;  break;   /* half d + 32 int8                   */
    case ORC_Q4_K: e = 256; b = 144; break;   /* half d, half dmin, 12 + 128 bytes  */
    case ORC_Q5_K: e = 256; b = 176; break;   /* half d, half dmin, 12 + 32 + 128   */
    case ORC_Q6_K: e = 256; b = 210; break;   /* 128 + 64 + 16 + half d             */
    case ORC_Q8_1: e = 32;  b = 36;  break;   /* half d, half s, 32 int8            */
    default: return ORC_ERR_TYPE;
    }
    if (block_elems) *block_elems = e;
    if (block_bytes) *block_bytes = b;
    return ORC_OK;
}

int orc_dots_per_block(int type) {
    switch (type) {
    case ORC_Q4_0: case ORC_Q4_1: case ORC_Q5_0: case ORC_Q5_1: return 1;
    case ORC_Q8_0: return 1;
    case ORC_Q4_K: case ORC_Q5_K: return 16;
    case ORC_Q6_K: return 16;
    default: return ORC_ERR_TYPE;
    }
}

/* ------------------------------------------------------------------------ */
/* q8_1 activation quantization [MMVQ §激活的量化]                           */
/* ------------------------------------------------------------------------ */
/* Readings taken here:
 *  - s is d*sum(q) as the struct comment and the prose describe it, formed
 *    as an fp32 product of the fp32 d and the exact integer sum, then
 *    rounded to fp16 (the printed kernel stores the float sum of x instead;
 *    the integer form is the one the struct documents and it does not
 *    depend on a reduction order).
 *  - q is formed with the fp32 d (before it is rounded to fp16), with C
 *    roundf (ties away from zero).
 *  - a block whose fp32 d is zero (amax == 0, or amax so small that
 *    amax/127 underflows to zero) gets q = 0, extending the amax == 0 guard
 *    of the printed kernel to the underflow case.
 *  - fp16 stores round to nearest even.
 */
int orc_quantize_q8_1(const float *x, int64_t K, int64_t n, int64_t ldx,
                      uint8_t *y_q) {
    if (!x || !y_q) return ORC_ERR_NULL;
    if (K <= 0 || K % 32 != 0 || n < 1 || ldx < K) return ORC_ERR_SHAPE;
    const int64_t nb = K / 32;
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + j * ldx + 32 * b;
            uint8_t *blk = y_q + (j * nb + b) * 36;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                const float ax = fabsf(xb[i]);
                if (ax > amax) amax = ax;
            }
            const float d = amax / 127.0f;
            int sumq = 0;
            for (int i = 0; i < 32; ++i) {
                const int q = (d == 0.0f) ? 0 : (int)roundf(xb[i] / d);
                blk[4 + i] = (uint8_t)(int8_t)q;
                sumq += q;
            }
            const float s = d * (float)sumq;
            wr16(blk + 0, orc_f32_to_f16(d));
            wr16(blk + 2, orc_f32_to_f16(s));
        }
    }
    return ORC_OK;
}

/* q8_1 field access: block b of one column. */
static double q8_d(const uint8_t *col, int64_t b) { return orc_f16_to_f64(rd16(col + 36 * b + 0)); }
static double q8_s(const uint8_t *col, int64_t b) { return orc_f16_to_f64(rd16(col + 36 * b + 2)); }
static int q8_q(const uint8_t *col, int64_t b, int i) { return (int8_t)col[36 * b + 4 + i]; }

int orc_dequantize_q8_1(const uint8_t *y_q, int64_t K, double *y) {
    if (!y_q || !y) return ORC_ERR_NULL;
    if (K <= 0 || K % 32 != 0) return ORC_ERR_SHAPE;
    for (int64_t e = 0; e < K; ++e) y[e] = q8_d(y_q, e / 32) * q8_q(y_q, e / 32, (int)(e % 32));
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Weight formats: the code of element e of one block                        */
/* ------------------------------------------------------------------------ */

/* Q4_0 [MMVQ §权重的排法, §一次 vec_dot 的解剖]: bytes 0-1 fp16 d, bytes
 * 2..17 qs. Reading: the low nibble of qs[j] is element j and the high
 * nibble is element j+16 (the printed dot pairs the low nibbles of a qs
 * word with activation word i and the high nibbles with word i + 4).
 * Weight value d*(q - 8). */
static int q4_0_code(const uint8_t *blk, int e) {
    const uint8_t *qs = blk + 2;
    return e < 16 ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);
}

/* Q4_1, Q5_0, Q5_1 [MMVQ §权重的排法 (old-style blocks of 32 weights, Q5_1
 * named among them); GGUF16 §16.1.1 (type ids 3, 6, 7)]. The pages name
 * these formats without their layouts; the layouts here are readings of the
 * published GGUF block definitions, field by field:
 *   Q4_1: fp16 d @0, fp16 m @2, qs[16] @4; weight d*q + m.
 *   Q5_0: fp16 d @0, qh (4 bytes, little-endian 32-bit word) @2, qs[16] @6;
 *         weight d*(q - 16).
 *   Q5_1: fp16 d @0, fp16 m @2, qh @4, qs[16] @8; weight d*q + m.
 * Low 4 bits of element e as in Q4_0 (the low nibble of qs[e] for e < 16,
 * the high nibble of qs[e - 16] above); the 5-bit formats take bit e of qh
 * as bit 4 of the code. */
static int nib_code(const uint8_t *qs, int e) { return e < 16 ? (qs[e] & 0x0F) : (qs[e - 16] >> 4); }
static int qh_bit(const uint8_t *qh, int e) { return (qh[e / 8] >> (e % 8)) & 1; }
static int q4_1_code(const uint8_t *blk, int e) { return nib_code(blk + 4, e); }
static int q5_0_code(const uint8_t *blk, int e) { return nib_code(blk + 6, e) | (qh_bit(blk + 2, e) << 4); }
static int q5_1_code(const uint8_t *blk, int e) { return nib_code(blk + 8, e) | (qh_bit(blk + 4, e) << 4); }

/* Q8_0 [LLM §量化格式 (format table: 8-bit, 34 bytes per 32 weights);
 * MMVQ §权重的排法 (old-style blocks: one fp16 scale for 32 codes)]. The
 * pages give the size and the block shape, not the struct. Reading: fp16 d
 * at bytes 0-1, 32 signed 8-bit codes at bytes 2..33 (element e = byte 2+e),
 * symmetric, no zero point. Weight value d*q. */
static int q8_0_code(const uint8_t *blk, int e) { return (int8_t)blk[2 + e]; }

/* Q4_K [GGUF16 §16.1.2, §16.2.1]: bytes 0-1 fp16 d, 2-3 fp16 dmin,
 * 4..15 the packed scales, 16..143 qs (the field order of the struct on the
 * GGUF16 page; the MMVQ page lists the fields in another order, read as a
 * garbled listing). Element e lies in sub-block t = e/32; the row decoder
 * walks 64-element chunks c, taking the low nibbles of qs[32c..32c+31] for
 * sub-block 2c and the high nibbles for sub-block 2c+1. Weight value
 * d*sc_t*q - dmin*m_t. */
static int q4_k_code(const uint8_t *blk, int e) {
    const uint8_t *qs = blk + 16;
    const int t = e / 32, l = e % 32, c = t / 2;
    const uint8_t byte = qs[32 * c + l];
    return (t % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Q4_K 6-bit scale/min unpack. The pages name the unpack routine without
 * printing it, and print a branch-free fragment that builds two 16-bit
 * words from three 16-bit scale words (s0, s2, s4) and a mask hi = -(j>=2)
 * for sub-block pair j. Reading s0, s2, s4 as the little-endian 16-bit
 * words jm, jm+2 and jm+4 of the 12 scale bytes (jm = j & 1), the fragment
 * gives, for sub-block t with scale bytes B[0..11]:
 *   t < 4 : sc = B[t] & 63,                  m = B[t+4] & 63
 *   t >= 4: sc = (B[t+4] & 15) | (B[t-4] >> 6) << 4,
 *           m  = (B[t+4] >> 4) | (B[t]   >> 6) << 4
 * [MMVQ §一次 vec_dot 的解剖 (the Q4_K scale fragment)]. */
void orc_q4_k_scale_min(const uint8_t *B, int t, int *sc, int *m) {
    if (t < 4) {
        *sc = B[t] & 63;
        *m = B[t + 4] & 63;
    } else {
        *sc = (B[t + 4] & 15) | ((B[t - 4] >> 6) << 4);
        *m = (B[t + 4] >> 4) | ((B[t] >> 6) << 4);
    }
}

/* Q6_K [MMVQ §dp4a, §一次 vec_dot 的解剖]: 256 weights, 16 sub-blocks of 16,
 * 6-bit codes stored as 4 low bits plus 2 high bits, offset -32, one int8
 * scale per sub-block, 210 bytes. The pages fix the size, the bit split and
 * that the high bits of the element held in a byte's high nibble sit four
 * bits above those of the low-nibble element; they do not print the struct.
 * Layout taken: ql[128] at 0, qh[64] at 128, int8 sc[16] at 192, fp16 d at
 * 208. Element e = 128h + 32g + l (h in 0..1, g in 0..3, l in 0..31):
 *   low 4 bits : g=0 ql[64h+l] & 15, g=1 ql[64h+32+l] & 15,
 *                g=2 ql[64h+l] >> 4, g=3 ql[64h+32+l] >> 4
 *   high 2 bits: (qh[32h+l] >> 2g) & 3
 *   sub-block  : e/16 = 8h + 2g + l/16
 * Weight value d*sc[e/16]*(q - 32). */
static int q6_k_code(const uint8_t *blk, int e) {
    const uint8_t *ql = blk, *qh = blk + 128;
    const int h = e / 128, g = (e % 128) / 32, l = e % 32;
    const uint8_t lbyte = ql[64 * h + 32 * (g % 2) + l];
    const int low = (g < 2) ? (lbyte & 0x0F) : (lbyte >> 4);
    const int high = (qh[32 * h + l] >> (2 * g)) & 3;
    return low | (high << 4);
}
static int q6_k_scale(const uint8_t *blk, int s) { return (int8_t)blk[192 + s]; }

/* Q5_K [MMVQ §激活的量化 (named among the min-term formats); GGUF16
 * §16.1.1 (type id 13)]. The pages name the format without its layout; the
 * layout is a reading of the published GGUF block definition: fp16 d @0,
 * fp16 dmin @2, the 12 packed scale/min bytes of Q4_K @4, qh[32] @16,
 * qs[128] @48, 176 bytes. Element e of sub-block t = e/32 (l = e%32, chunk
 * c = t/2): low 4 bits as in Q4_K (low or high nibble of qs[32c + l]), bit 4
 * = bit t of qh[l]. Weight value d*sc_t*q - dmin*m_t, q in 0..31. */
static int q5_k_code(const uint8_t *blk, int e) {
    const uint8_t *qh = blk + 16, *qs = blk + 48;
    const int t = e / 32, l = e % 32, c = t / 2;
    const uint8_t byte = qs[32 * c + l];
    const int low = (t % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return low | (((qh[l] >> t) & 1) << 4);
}

int orc_dequantize_row(int type, const uint8_t *row, int64_t K, double *w) {
    int qk, bb;
    if (!row || !w) return ORC_ERR_NULL;
    if (orc_type_info(type, &qk, &bb) != ORC_OK || type == ORC_Q8_1) return ORC_ERR_TYPE;
    if (K <= 0 || K % qk != 0) return ORC_ERR_SHAPE;
    for (int64_t e = 0; e < K; ++e) {
        const uint8_t *blk = row + (e / qk) * bb;
        const int i = (int)(e % qk);
        if (type == ORC_Q4_0) {
            w[e] = orc_f16_to_f64(rd16(blk)) * (q4_0_code(blk, i) - 8);
        } else if (type == ORC_Q4_1) {
            w[e] = orc_f16_to_f64(rd16(blk)) * q4_1_code(blk, i) + orc_f16_to_f64(rd16(blk + 2));
        } else if (type == ORC_Q5_0) {
            w[e] = orc_f16_to_f64(rd16(blk)) * (q5_0_code(blk, i) - 16);
        } else if (type == ORC_Q5_1) {
            w[e] = orc_f16_to_f64(rd16(blk)) * q5_1_code(blk, i) + orc_f16_to_f64(rd16(blk + 2));
        } else if (type == ORC_Q5_K) {
            int sc, m;
            orc_q4_k_scale_min(blk + 4, i / 32, &sc, &m);
            w[e] = orc_f16_to_f64(rd16(blk)) * sc * q5_k_code(blk, i)
                 - orc_f16_to_f64(rd16(blk + 2)) * m;
        } else if (type == ORC_Q8_0) {
            w[e] = orc_f16_to_f64(rd16(blk)) * q8_0_code(blk, i);
        } else if (type == ORC_Q4_K) {
            int sc, m;
            orc_q4_k_scale_min(blk + 4, i / 32, &sc, &m);
            w[e] = orc_f16_to_f64(rd16(blk)) * sc * q4_k_code(blk, i)
                 - orc_f16_to_f64(rd16(blk + 2)) * m;
        } else {
            w[e] = orc_f16_to_f64(rd16(blk + 208)) * q6_k_scale(blk, i / 16)
                 * (q6_k_code(blk, i) - 32);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Block dots and scale application                                          */
/* ------------------------------------------------------------------------ */
/* One weight block (qk elements) against the matching q8_1 blocks of one
 * activation column. Adds the block's contribution to *acc, the absolute
 * values of its terms to *mag, and writes its integer dots to dots (if not
 * NULL). qb is the index of the first q8_1 block of this weight block
 * (the weight block index times qk/32 [MMVQ §kernel 的形状]). */

/* Q4_0: isum = sum q*qy; contribution d_w*(d8*isum - 8*s)
 * [MMVQ §一次 vec_dot 的解剖]. */
static void block_q4_0(const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                       double *acc, double *mag, int32_t *dots) {
    int isum = 0;
    for (int e = 0; e < 32; ++e) isum += q4_0_code(blk, e) * q8_q(ycol, qb, e);
    const double dw = orc_f16_to_f64(rd16(blk));
    const double t1 = dw * q8_d(ycol, qb) * isum;
    const double t2 = 8.0 * dw * q8_s(ycol, qb);
    *acc += t1 - t2;
    *mag += fabs(t1) + fabs(t2);
    if (dots) dots[0] = isum;
}

/* Q4_1, Q5_1: isum = sum q*qy; contribution d*d8*isum + m*s: the offset
 * term takes the q8_1 block's stored s (fp16 d8*sum(qy)), as Q4_0 does for
 * its zero point; the pages give no dot for these formats, and s exists in
 * q8_1 for exactly this term [MMVQ §激活的量化].
 * Q5_0: contribution d*(d8*isum - 16*s) (zero point 16 of the 5-bit code,
 * as Q4_0's 8 of the 4-bit one). */
static void block_legacy(int type, const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                         double *acc, double *mag, int32_t *dots) {
    int isum = 0;
    for (int e = 0; e < 32; ++e) {
        const int q = type == ORC_Q4_1 ? q4_1_code(blk, e) : type == ORC_Q5_0 ? q5_0_code(blk, e)
                                                                            : q5_1_code(blk, e);
        isum += q * q8_q(ycol, qb, e);
    }
    const double d = orc_f16_to_f64(rd16(blk));
    const double t1 = d * q8_d(ycol, qb) * isum;
    const double t2 = type == ORC_Q5_0 ? -16.0 * d * q8_s(ycol, qb)
                                       : orc_f16_to_f64(rd16(blk + 2)) * q8_s(ycol, qb);
    *acc += t1 + t2;
    *mag += fabs(t1) + fabs(t2);
    if (dots) dots[0] = isum;
}

/* Q8_0: isum = sum q*qy; contribution d_w*d8*isum (symmetric codes: no
 * zero-point or min term). */
static void block_q8_0(const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                       double *acc, double *mag, int32_t *dots) {
    int isum = 0;
    for (int e = 0; e < 32; ++e) isum += q8_0_code(blk, e) * q8_q(ycol, qb, e);
    const double t = orc_f16_to_f64(rd16(blk)) * q8_d(ycol, qb) * isum;
    *acc += t;
    *mag += fabs(t);
    if (dots) dots[0] = isum;
}

/* Q4_K (and Q5_K, whose codes come from another code function): per
 * sub-block t, dot1 = sum q*qy, dot2 = sum qy over its 32 elements;
 * contribution d*sc*d8*dot1 - dmin*m*d8*dot2, the min term kept apart
 * [MMVQ §一次 vec_dot 的解剖]. Sub-block t pairs with q8_1 block qb + t.
 * The magnitude (the tolerance's error scale) sums both terms over each
 * 16-element half of the sub-block: an evaluation may scale and sum the
 * halves' partial dots in fp32 before they meet, and where the halves
 * cancel, those partials exceed the sub-block's terms. */
static void block_k_min(const uint8_t *blk, const uint8_t *ycol, int64_t qb, double *acc, double *mag,
                        int32_t *dots, int (*code)(const uint8_t *, int)) {
    const double d = orc_f16_to_f64(rd16(blk));
    const double dmin = orc_f16_to_f64(rd16(blk + 2));
    for (int t = 0; t < 8; ++t) {
        int sc, m, dot1 = 0, dot2 = 0, half1[2] = {0, 0}, half2[2] = {0, 0};
        orc_q4_k_scale_min(blk + 4, t, &sc, &m);
        for (int l = 0; l < 32; ++l) {
            const int qy = q8_q(ycol, qb + t, l);
            dot1 += code(blk, 32 * t + l) * qy;
            dot2 += qy;
            half1[l / 16] += code(blk, 32 * t + l) * qy;
            half2[l / 16] += qy;
        }
        const double d8 = q8_d(ycol, qb + t);
        const double t1 = d * sc * d8 * dot1;
        const double t2 = dmin * m * d8 * dot2;
        *acc += t1 - t2;
        for (int h = 0; h < 2; ++h) *mag += fabs(d * sc * d8 * half1[h]) + fabs(dmin * m * d8 * half2[h]);
        if (dots) { dots[t] = dot1; dots[8 + t] = dot2; }
    }
}

static void block_q4_k(const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                       double *acc, double *mag, int32_t *dots) {
    block_k_min(blk, ycol, qb, acc, mag, dots, q4_k_code);
}

/* Q5_K: as Q4_K with the 5-bit codes: per sub-block t, dot1 = sum q*qy,
 * dot2 = sum qy; contribution d*sc*d8*dot1 - dmin*m*d8*dot2. */
static void block_q5_k(const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                       double *acc, double *mag, int32_t *dots) {
    block_k_min(blk, ycol, qb, acc, mag, dots, q5_k_code);
}

/* Q6_K: per sub-block s of 16, isum_s = sum (q - 32)*qy; contribution
 * d*sc_s*d8*isum_s [MMVQ §dp4a]. Sub-blocks 2b and 2b+1 share q8_1 block
 * qb + b. */
static void block_q6_k(const uint8_t *blk, const uint8_t *ycol, int64_t qb,
                       double *acc, double *mag, int32_t *dots) {
    const double d = orc_f16_to_f64(rd16(blk + 208));
    for (int s = 0; s < 16; ++s) {
        const int64_t yb = qb + s / 2;
        int isum = 0;
        for (int i = 0; i < 16; ++i) {
            const int e = 16 * s + i;
            isum += (q6_k_code(blk, e) - 32) * q8_q(ycol, yb, e % 32);
        }
        const double t = d * q6_k_scale(blk, s) * q8_d(ycol, yb) * isum;
        *acc += t;
        *mag += fabs(t);
        if (dots) dots[s] = isum;
    }
}

/* One row of W (nb weight blocks) against one q8_1 column. */
static void row_dot(const uint8_t *Wrow, int type, int64_t nb, int bb, int qk,
                    const uint8_t *ycol, double *acc, double *mag, int32_t *dots) {
    const int nd = orc_dots_per_block(type);
    *acc = 0.0;
    *mag = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = Wrow + b * bb;
        const int64_t qb = b * (qk / 32);
        int32_t *dp = dots ? dots + b * nd : NULL;
        if (type == ORC_Q4_0) block_q4_0(blk, ycol, qb, acc, mag, dp);
        else if (type == ORC_Q4_1 || type == ORC_Q5_0 || type == ORC_Q5_1)
            block_legacy(type, blk, ycol, qb, acc, mag, dp);
        else if (type == ORC_Q8_0) block_q8_0(blk, ycol, qb, acc, mag, dp);
        else if (type == ORC_Q4_K) block_q4_k(blk, ycol, qb, acc, mag, dp);
        else if (type == ORC_Q5_K) block_q5_k(blk, ycol, qb, acc, mag, dp);
        else block_q6_k(blk, ycol, qb, acc, mag, dp);
    }
}

static int gemv_args_ok(const uint8_t *W, int type, int64_t M, int64_t K,
                        const uint8_t *y_q, int64_t n, int *qk, int *bb) {
    if (!W || !y_q) return ORC_ERR_NULL;
    if (orc_type_info(type, qk, bb) != ORC_OK || type == ORC_Q8_1) return ORC_ERR_TYPE;
    if (M < 1 || K <= 0 || K % *qk != 0 || n < 1) return ORC_ERR_SHAPE;
    return ORC_OK;
}

int orc_mmvq_rows(const uint8_t *W, int type, int64_t M, int64_t K,
                  const uint8_t *y_q, int64_t n, int64_t r0, int64_t r1,
                  double *out, double *mag, int32_t *dots) {
    int qk, bb;
    int rc = gemv_args_ok(W, type, M, K, y_q, n, &qk, &bb);
    if (rc) return rc;
    if (!out) return ORC_ERR_NULL;
    if (r0 < 0 || r1 > M || r0 > r1) return ORC_ERR_SHAPE;
    const int64_t nb = K / qk;              /* weight blocks per row */
    const int64_t ycol_bytes = (K / 32) * 36;
    const int nd = orc_dots_per_block(type);
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t r = r0; r < r1; ++r) {
            double acc, mg;
            row_dot(W + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &acc, &mg,
                    dots ? dots + (j * M + r) * nb * nd : NULL);
            out[j * M + r] = acc;
            if (mag) mag[j * M + r] = mg;
        }
    }
    return ORC_OK;
}

int orc_mmvq(const uint8_t *W, int type, int64_t M, int64_t K,
             const uint8_t *y_q, int64_t n, double *out, double *mag,
             int32_t *dots) {
    return orc_mmvq_rows(W, type, M, K, y_q, n, 0, M, out, mag, dots);
}

/* ------------------------------------------------------------------------ */
/* GLU epilogue [MMVQ §融合]                                                 */
/* ------------------------------------------------------------------------ */
/* The page's epilogue switch names the GLU ops and the device functions
 * that apply them, without their bodies. Readings (parity unpinned against
 * the pages, which fix none of these formulas):
 *  - SWIGLU: silu(g)*u with silu(z) = z*sigmoid(z), the Swish-1 / SiLU of
 *    the GLU-variants literature (Shazeer, "GLU Variants Improve
 *    Transformer", 2020).
 *  - GEGLU: gelu(g)*u with gelu in the tanh form published with GELU
 *    (Hendrycks and Gimpel, "Gaussian Error Linear Units", 2016):
 *    0.5*z*(1 + tanh(sqrt(2/pi)*(z + 0.044715*z^3))). The op list on the
 *    page has a single GEGLU entry; the operator set it comes from keeps
 *    the exact erf form as a separate op, so the plain entry is read as the
 *    tanh form.
 *  - SWIGLU_OAI: the clamped SwiGLU published with the gpt-oss models,
 *    g'*sigmoid(alpha*g')*(u' + 1) with g' = min(g, limit),
 *    u' = clamp(u, -limit, limit) and that publication's constants
 *    alpha = 1.702, limit = 7. The page calls it with the gate and the up
 *    value only, so the constants are the op's own, not parameters.
 *  - SWIGLU_CLAMP: the page passes the caller's glu_limit; taken as the same
 *    clamps around a plain SwiGLU, silu(g')*u'. No public definition is
 *    known to this reading beyond the call. */
#define ORC_OAI_ALPHA 1.702
#define ORC_OAI_LIMIT 7.0

static double silu(double z) { return z / (1.0 + exp(-z)); }

static double gelu_tanh(double z) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

int orc_glu(int glu_op, double g, double u, double limit, double *out) {
    if (!out) return ORC_ERR_NULL;
    switch (glu_op) {
    case ORC_GLU_PLAIN: *out = g * u; break;
    case ORC_GLU_SWIGLU: *out = silu(g) * u; break;
    case ORC_GLU_GEGLU: *out = gelu_tanh(g) * u; break;
    case ORC_GLU_SWIGLU_OAI: {
        const double gc = g < ORC_OAI_LIMIT ? g : ORC_OAI_LIMIT;
        const double uc = u < -ORC_OAI_LIMIT ? -ORC_OAI_LIMIT : (u > ORC_OAI_LIMIT ? ORC_OAI_LIMIT : u);
        *out = gc / (1.0 + exp(-ORC_OAI_ALPHA * gc)) * (uc + 1.0);
        break;
    }
    case ORC_GLU_SWIGLU_CLAMP: {
        const double gc = g < limit ? g : limit;
        const double uc = u < -limit ? -limit : (u > limit ? limit : u);
        *out = silu(gc) * uc;
        break;
    }
    default: return ORC_ERR_TYPE;
    }
    return ORC_OK;
}

/* Ops the plain fused calls take: those with no caller parameter. */
static int valid_glu(int glu_op) {
    return glu_op == ORC_GLU_PLAIN || glu_op == ORC_GLU_SWIGLU || glu_op == ORC_GLU_GEGLU ||
           glu_op == ORC_GLU_SWIGLU_OAI;
}

int orc_mmvq_glu(const uint8_t *W_gate, const uint8_t *W_up, int type,
                 int64_t M, int64_t K, const uint8_t *y_q, int64_t n,
                 int glu_op, double *out) {
    int qk, bb;
    int rc = gemv_args_ok(W_gate, type, M, K, y_q, n, &qk, &bb);
    if (rc) return rc;
    if (!W_up || !out) return ORC_ERR_NULL;
    if (!valid_glu(glu_op)) return ORC_ERR_TYPE;
    const int64_t nb = K / qk;
    const int64_t ycol_bytes = (K / 32) * 36;
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t r = 0; r < M; ++r) {
            double g, u, mg;
            row_dot(W_gate + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &g, &mg, NULL);
            row_dot(W_up + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &u, &mg, NULL);
            rc = orc_glu(glu_op, g, u, 0.0, &out[j * M + r]);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Full fused epilogue [MMVQ §融合]                                           */
/* ------------------------------------------------------------------------ */
/* One output: raw dots of the up (and gate) row, then the epilogue, with
 * the scales and biases of expert e (0 outside the expert-indexed form). */
static int epilogue_one(const orc_epilogue *epi, int has_gate, int e, int64_t M, int64_t r,
                        double up, double gate, double *out) {
    if (!epi) {
        *out = has_gate ? gate * up : up;
        return ORC_OK;
    }
    double u = up;
    if (epi->up_scale) u *= epi->up_scale[e];
    if (epi->up_bias) u += epi->up_bias[(int64_t)e * M + r];
    if (!has_gate) {
        *out = u;
        return ORC_OK;
    }
    double g = gate;
    if (epi->gate_scale) g *= epi->gate_scale[e];
    if (epi->gate_bias) g += epi->gate_bias[(int64_t)e * M + r];
    return orc_glu(epi->glu_op, g, u, epi->limit, out);
}

int orc_mmvq_ex(const uint8_t *W_up, const uint8_t *W_gate, int type,
                int64_t M, int64_t K, const uint8_t *y_q, int64_t n,
                const orc_epilogue *epi, double *out) {
    int qk, bb;
    int rc = gemv_args_ok(W_up, type, M, K, y_q, n, &qk, &bb);
    if (rc) return rc;
    if (!out) return ORC_ERR_NULL;
    const int64_t nb = K / qk;
    const int64_t ycol_bytes = (K / 32) * 36;
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t r = 0; r < M; ++r) {
            double u, g = 0.0, mag;
            row_dot(W_up + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &u, &mag, NULL);
            if (W_gate) row_dot(W_gate + r * nb * bb, type, nb, bb, qk, y_q + j * ycol_bytes, &g, &mag, NULL);
            rc = epilogue_one(epi, W_gate != NULL, 0, M, r, u, g, &out[j * M + r]);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert-indexed product [MMVQ §MoE, §正确性上的几个坑]                      */
/* ------------------------------------------------------------------------ */
/* Reading: token t's one q8_1 column is shared by its top_k slots, and the
 * output is token-major, then slot, then row. */
static int id_args_ok(const uint8_t *W, int64_t expert_stride, int n_experts,
                      int type, int64_t M, int64_t K, int64_t n_tokens,
                      const int32_t *ids, int top_k) {
    int qk, bb;
    if (!W || !ids) return ORC_ERR_NULL;
    if (orc_type_info(type, &qk, &bb) != ORC_OK || type == ORC_Q8_1) return ORC_ERR_TYPE;
    if (n_experts < 1 || top_k < 1 || top_k > n_experts || n_tokens < 1 || M < 1 ||
        K <= 0 || K % qk != 0 || expert_stride < M * (K / qk) * bb)
        return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n_tokens * top_k; ++i)
        if (ids[i] < 0 || ids[i] >= n_experts) return ORC_ERR_ID;
    return ORC_OK;
}

int orc_mmvq_id(const uint8_t *W, int64_t expert_stride, int n_experts,
                int type, int64_t M, int64_t K, const uint8_t *y_q,
                int64_t n_tokens, const int32_t *ids, int top_k,
                double *out, double *mag) {
    if (!y_q || !out) return ORC_ERR_NULL;
    int rc = id_args_ok(W, expert_stride, n_experts, type, M, K, n_tokens, ids, top_k);
    if (rc) return rc;
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int k = 0; k < top_k; ++k) {
            const int64_t slot = t * top_k + k;
            const uint8_t *We = W + (int64_t)ids[slot] * expert_stride;
            rc = orc_mmvq(We, type, M, K, y_q + t * (K / 32) * 36, 1,
                          out + slot * M, mag ? mag + slot * M : NULL, NULL);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

int orc_mmvq_id_glu(const uint8_t *W_gate, const uint8_t *W_up,
                    int64_t expert_stride, int n_experts, int type,
                    int64_t M, int64_t K, const uint8_t *y_q,
                    int64_t n_tokens, const int32_t *ids, int top_k,
                    int glu_op, double *out) {
    if (!W_up || !y_q || !out) return ORC_ERR_NULL;
    if (!valid_glu(glu_op)) return ORC_ERR_TYPE;
    int rc = id_args_ok(W_gate, expert_stride, n_experts, type, M, K, n_tokens, ids, top_k);
    if (rc) return rc;
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int k = 0; k < top_k; ++k) {
            const int64_t slot = t * top_k + k;
            const int64_t off = (int64_t)ids[slot] * expert_stride;
            rc = orc_mmvq_glu(W_gate + off, W_up + off, type, M, K,
                              y_q + t * (K / 32) * 36, 1, glu_op, out + slot * M);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* Expert-indexed epilogue form; the shared expert (an extra grid slice on
 * the pages) applies to every token with the GLU only [MMVQ §融合]. */
int orc_mmvq_id_ex(const uint8_t *W_up, const uint8_t *W_gate,
                   int64_t expert_stride, int n_experts, int type,
                   int64_t M, int64_t K, const uint8_t *y_q,
                   int64_t n_tokens, const int32_t *ids, int top_k,
                   const orc_epilogue *epi, const uint8_t *shared_up,
                   const uint8_t *shared_gate, double *shared_out,
                   double *out) {
    if (!y_q || !out) return ORC_ERR_NULL;
    if (shared_up && !shared_out) return ORC_ERR_NULL;
    int rc = id_args_ok(W_up, expert_stride, n_experts, type, M, K, n_tokens, ids, top_k);
    if (rc) return rc;
    int qk, bb;
    orc_type_info(type, &qk, &bb);
    const int64_t nb = K / qk;
    const int64_t ycol_bytes = (K / 32) * 36;
    for (int64_t t = 0; t < n_tokens; ++t) {
        const uint8_t *yt = y_q + t * ycol_bytes;
        for (int k = 0; k < top_k; ++k) {
            const int64_t slot = t * top_k + k;
            const int e = ids[slot];
            const int64_t off = (int64_t)e * expert_stride;
            for (int64_t r = 0; r < M; ++r) {
                double u, g = 0.0, mag;
                row_dot(W_up + off + r * nb * bb, type, nb, bb, qk, yt, &u, &mag, NULL);
                if (W_gate) row_dot(W_gate + off + r * nb * bb, type, nb, bb, qk, yt, &g, &mag, NULL);
                rc = epilogue_one(epi, W_gate != NULL, e, M, r, u, g, &out[slot * M + r]);
                if (rc) return rc;
            }
        }
        if (shared_up) {
            for (int64_t r = 0; r < M; ++r) {
                double u, g = 0.0, mag;
                row_dot(shared_up + r * nb * bb, type, nb, bb, qk, yt, &u, &mag, NULL);
                if (shared_gate) {
                    row_dot(shared_gate + r * nb * bb, type, nb, bb, qk, yt, &g, &mag, NULL);
                    rc = orc_glu(epi ? epi->glu_op : ORC_GLU_PLAIN, g, u, epi ? epi->limit : 0.0,
                                 &shared_out[t * M + r]);
                    if (rc) return rc;
                } else {
                    shared_out[t * M + r] = u;
                }
            }
        }
    }
    return ORC_OK;
}
