/*
 * oracle_drive.c - runs every oracle entry point on small random inputs and
 * on the documented error paths, for a build under the address and
 * undefined-behaviour sanitizers (the oracle is plain C; this driver adds
 * no arithmetic of its own, it only calls the oracle and checks return
 * codes). Exits non-zero on a failing return code; the sanitizers abort on
 * any out-of-bounds access, use of uninitialized heap, overflow of a signed
 * integer or invalid shift.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/mmvq_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}
static float rnd_f(float scale) { return ((float)(rnd() % 2000001) / 1000000.0f - 1.0f) * scale; }

static int fails = 0;
#define CHECK(expr, want)                                                              \
    do {                                                                               \
        int rc_ = (expr);                                                              \
        if (rc_ != (want)) {                                                           \
            printf("FAIL line %d: %s returned %d, expected %d\n", __LINE__, #expr, rc_, \
                   (want));                                                            \
            ++fails;                                                                   \
        }                                                                              \
    } while (0)

/* exactly-sized heap buffers, so a one-past read is caught */
static uint8_t *weights(int type, int64_t M, int64_t K) {
    int qk, bb;
    orc_type_info(type, &qk, &bb);
    const size_t n = (size_t)(M * (K / qk) * bb);
    uint8_t *w = malloc(n);
    for (size_t i = 0; i < n; ++i) w[i] = (uint8_t)rnd();
    /* finite fp16 block scales: clear the top exponent bit of every scale field */
    for (int64_t b = 0; b < M * (K / qk); ++b) {
        uint8_t *blk = w + b * bb;
        if (type == ORC_Q4_K) { blk[1] &= 0x3B; blk[3] &= 0x3B; }
        else if (type == ORC_Q6_K) blk[209] &= 0x3B;
        else blk[1] &= 0x3B;
    }
    return w;
}

static void one_shape(int type, int64_t M, int64_t K, int64_t n) {
    float *x = malloc((size_t)(n * K) * sizeof(float));
    for (int64_t i = 0; i < n * K; ++i) x[i] = rnd_f(i % 97 == 0 ? 1e4f : 2.0f);
    uint8_t *y = malloc((size_t)(n * (K / 32) * 36));
    CHECK(orc_quantize_q8_1(x, K, n, K, y), ORC_OK);
    uint8_t *W = weights(type, M, K), *Wg = weights(type, M, K);
    int qk, bb;
    orc_type_info(type, &qk, &bb);
    const int nd = orc_dots_per_block(type);
    double *out = malloc((size_t)(n * M) * sizeof(double));
    double *mag = malloc((size_t)(n * M) * sizeof(double));
    int32_t *dots = malloc((size_t)(n * M * (K / qk) * nd) * sizeof(int32_t));
    CHECK(orc_mmvq(W, type, M, K, y, n, out, mag, dots), ORC_OK);
    CHECK(orc_mmvq_rows(W, type, M, K, y, n, M / 2, M, out, mag, NULL), ORC_OK);
    for (int op = 0; op <= 3; ++op) CHECK(orc_mmvq_glu(Wg, W, type, M, K, y, n, op, out), ORC_OK);
    CHECK(orc_mmvq_glu(Wg, W, type, M, K, y, n, ORC_GLU_SWIGLU_CLAMP, out), ORC_ERR_TYPE);
    double *bias = malloc((size_t)(3 * M) * sizeof(double)), scale[3] = {0.5, 1.0, 2.0};
    for (int64_t i = 0; i < 3 * M; ++i) bias[i] = rnd_f(1.0f);
    for (int op = 0; op <= 4; ++op) {
        orc_epilogue e = {bias, bias, scale, scale, op, 3.0};
        CHECK(orc_mmvq_ex(W, Wg, type, M, K, y, n, &e, out), ORC_OK);
        CHECK(orc_mmvq_ex(W, NULL, type, M, K, y, n, &e, out), ORC_OK);
    }
    /* expert-indexed: three experts back to back */
    const int64_t stride = M * (K / qk) * bb;
    uint8_t *E = malloc((size_t)(3 * stride)), *Eg = malloc((size_t)(3 * stride));
    for (int e = 0; e < 3; ++e) {
        uint8_t *a = weights(type, M, K), *g = weights(type, M, K);
        memcpy(E + e * stride, a, (size_t)stride);
        memcpy(Eg + e * stride, g, (size_t)stride);
        free(a);
        free(g);
    }
    int32_t ids[16];
    for (int i = 0; i < 2 * n; ++i) ids[i] = (int32_t)(rnd() % 3);
    double *oid = malloc((size_t)(2 * n * M) * sizeof(double)), *omag = malloc((size_t)(2 * n * M) * sizeof(double));
    double *sh = malloc((size_t)(n * M) * sizeof(double));
    CHECK(orc_mmvq_id(E, stride, 3, type, M, K, y, n, ids, 2, oid, omag), ORC_OK);
    CHECK(orc_mmvq_id_glu(Eg, E, stride, 3, type, M, K, y, n, ids, 2, ORC_GLU_SWIGLU, oid), ORC_OK);
    orc_epilogue e = {bias, bias, scale, scale, ORC_GLU_SWIGLU_OAI, 0.0};
    CHECK(orc_mmvq_id_ex(E, Eg, stride, 3, type, M, K, y, n, ids, 2, &e, W, Wg, sh, oid), ORC_OK);
    ids[0] = 3;
    CHECK(orc_mmvq_id(E, stride, 3, type, M, K, y, n, ids, 2, oid, omag), ORC_ERR_ID);
    double *row = malloc((size_t)K * sizeof(double)), *yd = malloc((size_t)K * sizeof(double));
    CHECK(orc_dequantize_row(type, W, K, row), ORC_OK);
    CHECK(orc_dequantize_q8_1(y, K, yd), ORC_OK);
    free(x); free(y); free(W); free(Wg); free(out); free(mag); free(dots); free(bias);
    free(E); free(Eg); free(oid); free(omag); free(sh); free(row); free(yd);
}

int main(void) {
    const int types[8] = {ORC_Q4_0, ORC_Q8_0, ORC_Q4_K, ORC_Q6_K, ORC_Q4_1, ORC_Q5_0, ORC_Q5_1, ORC_Q5_K};
    for (int t = 0; t < 8; ++t) {
        int qk, bb;
        orc_type_info(types[t], &qk, &bb);
        const int64_t Ks[3] = {qk, 2 * qk, 4 * qk > 256 ? 4 * qk : 256};
        for (int k = 0; k < 3; ++k)
            for (int64_t M = 1; M <= 5; M += 2)
                for (int64_t n = 1; n <= 8; n += 3) one_shape(types[t], M, Ks[k], n);
    }
    /* q8_1 edge blocks: zeros, subnormals, huge values, exact ties */
    float x[128];
    uint8_t y[4 * 36];
    for (int i = 0; i < 32; ++i) { x[i] = 0.0f; x[32 + i] = 1e-40f * (float)(i - 16); x[64 + i] = 6e4f * (float)(i % 3 - 1); x[96 + i] = (float)(i - 16) + 0.5f; }
    CHECK(orc_quantize_q8_1(x, 128, 1, 128, y), ORC_OK);
    /* error paths */
    double d;
    CHECK(orc_mmvq(NULL, ORC_Q4_K, 1, 256, y, 1, &d, NULL, NULL), ORC_ERR_NULL);
    CHECK(orc_mmvq(y, 5, 1, 256, y, 1, &d, NULL, NULL), ORC_ERR_TYPE);
    CHECK(orc_mmvq(y, ORC_Q4_K, 1, 200, y, 1, &d, NULL, NULL), ORC_ERR_SHAPE);
    CHECK(orc_quantize_q8_1(x, 33, 1, 33, y), ORC_ERR_SHAPE);
    CHECK(orc_glu(9, 1.0, 1.0, 0.0, &d), ORC_ERR_TYPE);
    CHECK(orc_glu(1, 1.0, 1.0, 0.0, NULL), ORC_ERR_NULL);
    printf("%s: %d failure(s)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
