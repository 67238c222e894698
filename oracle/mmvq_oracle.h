/*
 * mmvq_oracle.h - plain CPU oracle for the decode-time quantized mat-vec (MMVQ).
 *
 * TEST INFRASTRUCTURE ONLY. This library exists to check the GPU library
 * against a slow, obviously correct definition. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. The product
 * path (include/mmvq.h and the HIP library) never links, loads or calls it,
 * and it shares no code, header, table or helper with the product.
 *
 * Citations (the reader has the pages, not this repository's notes):
 *   [MMVQ §X]   page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时一条量化权重
 *               如何被 dp4a 逐块点积" (pinghaoyang.com.cn), section X.
 *   [GGUF16 §X] page "GGUF 量化内幕：第16章 llama.cpp 量化代码架构"
 *               (cnblogs apachecn), section X.
 *   [LLM §X]    page "解构LLM：以llama.cpp分析模型推理过程" (laumy.tech),
 *               section X.
 *
 * What the oracle computes:
 *   1. q8_1 quantization of fp32 activations [MMVQ §激活的量化]: per 32
 *      values, d = amax/127 (fp32), q = roundf(x/d), stored as
 *      {fp16 d, fp16 s = d*sum(q), int8 q[32]}.
 *   2. The quantized mat-vec as the sum over weight blocks of
 *      (scale products) x (integer block dot), accumulated in fp64
 *      [MMVQ §一次 vec_dot 的解剖, §dp4a].
 *   3. The fused gate/up GLU epilogue [MMVQ §融合] and the expert-indexed
 *      mul_mat_id [MMVQ §MoE, §正确性上的几个坑].
 *   4. The full fused epilogue [MMVQ §融合]: per-matrix scales, biases, the
 *      GLU variants, and the shared expert of a MoE layer.
 *
 * Every function returns 0 on success or a negative ORC_ERR_* code, and
 * never aborts.
 */
#ifndef MMVQ_ORACLE_H
#define MMVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Type ids follow the ggml numbering [GGUF16 §16.1.1]. */
/* (Q8_0 is in the same enumeration, id 8.) */
#define ORC_Q4_0 2
#define ORC_Q4_1 3
#define ORC_Q5_0 6
#define ORC_Q5_1 7
#define ORC_Q8_0 8
#define ORC_Q8_1 9
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14

#define ORC_GLU_PLAIN        0 /* out = gate * up (the epilogue's default branch) */
#define ORC_GLU_SWIGLU       1 /* out = silu(gate) * up                          */
#define ORC_GLU_GEGLU        2 /* out = gelu(gate) * up, gelu in its tanh form    */
#define ORC_GLU_SWIGLU_OAI   3 /* out = g' * sigmoid(1.702*g') * (u' + 1), limit 7 */
#define ORC_GLU_SWIGLU_CLAMP 4 /* out = silu(g') * u', caller's limit             */
/* with g' = min(gate, limit), u' = min(max(up, -limit), limit). */

#define ORC_OK          0
#define ORC_ERR_NULL   -1
#define ORC_ERR_TYPE   -2
#define ORC_ERR_SHAPE  -3
#define ORC_ERR_ID     -6

/* IEEE 754 binary16 conversions, written from the format definition. */
uint16_t orc_f32_to_f16(float f);   /* round to nearest, ties to even */
double   orc_f16_to_f64(uint16_t h);

/* Elements and bytes per block: Q4_0 32/18, Q4_1 32/20, Q5_0 32/22,
 * Q5_1 32/24, Q8_0 32/34, Q4_K 256/144, Q5_K 256/176, Q6_K 256/210,
 * Q8_1 32/36. */
int orc_type_info(int type, int *block_elems, int *block_bytes);

/* Number of int32 dots the oracle reports per weight block:
 * Q4_0, Q4_1, Q5_0, Q5_1 and Q8_0 1 (the block dot sum(q*qy) of the unsigned
 * or signed codes), Q4_K and Q5_K 16 (dot1 of sub-blocks 0..7, then the
 * activation sums dot2 of sub-blocks 0..7), Q6_K 16 (one per sub-block). */
int orc_dots_per_block(int type);

/* x: n columns of K floats, column j at x + j*ldx. y_q: n*(K/32) blocks of
 * 36 bytes, column j at y_q + j*(K/32)*36. */
int orc_quantize_q8_1(const float *x, int64_t K, int64_t n, int64_t ldx,
                      uint8_t *y_q);

/* out[j*M + r] = sum over the blocks of row r of W against column j of y_q,
 * for rows r0 <= r < r1 only (other entries are left untouched).
 * mag (optional) receives, in the same layout, the sum of the absolute
 * values of every per-block term added into out.
 * dots (optional) receives the integer dots, at
 * dots[((j*M + r)*nblocks + b)*orc_dots_per_block(type) + i]. */
int orc_mmvq_rows(const uint8_t *W, int type, int64_t M, int64_t K,
                  const uint8_t *y_q, int64_t n, int64_t r0, int64_t r1,
                  double *out, double *mag, int32_t *dots);

/* All rows. */
int orc_mmvq(const uint8_t *W, int type, int64_t M, int64_t K,
             const uint8_t *y_q, int64_t n, double *out, double *mag,
             int32_t *dots);

/* out[j*M + r] = orc_glu(glu_op, g, u) with g = W_gate row r . y_j and
 * u = W_up row r . y_j. Ops that take no caller parameter only (PLAIN,
 * SWIGLU, GEGLU, SWIGLU_OAI); ORC_ERR_TYPE for SWIGLU_CLAMP, whose limit
 * only the epilogue form carries. */
int orc_mmvq_glu(const uint8_t *W_gate, const uint8_t *W_up, int type,
                 int64_t M, int64_t K, const uint8_t *y_q, int64_t n,
                 int glu_op, double *out);

/* Expert-indexed product: expert e's matrix starts at W + e*expert_stride.
 * ids holds n_tokens*top_k expert ids, token-major. For token t and slot k,
 * out[(t*top_k + k)*M + r] = row r of expert ids[t*top_k+k] . column t of
 * y_q. mag as for orc_mmvq. Returns ORC_ERR_ID for an id outside
 * 0..n_experts-1. */
int orc_mmvq_id(const uint8_t *W, int64_t expert_stride, int n_experts,
                int type, int64_t M, int64_t K, const uint8_t *y_q,
                int64_t n_tokens, const int32_t *ids, int top_k,
                double *out, double *mag);

int orc_mmvq_id_glu(const uint8_t *W_gate, const uint8_t *W_up,
                    int64_t expert_stride, int n_experts, int type,
                    int64_t M, int64_t K, const uint8_t *y_q,
                    int64_t n_tokens, const int32_t *ids, int top_k,
                    int glu_op, double *out);

/* The GLU of one gate value g and one up value u [MMVQ §融合]; limit is used
 * by SWIGLU_CLAMP only (SWIGLU_OAI has its own constants). ORC_ERR_TYPE for
 * an unknown op. */
int orc_glu(int glu_op, double g, double u, double limit, double *out);

/* Fused epilogue [MMVQ §融合], applied in the order the pages list it:
 * u = up_dot * up_scale + up_bias[r]; with a gate matrix,
 * g = gate_dot * gate_scale + gate_bias[r] and out = glu(g, u); without
 * one, out = u. Any pointer may be NULL (scale 1, bias 0). In the
 * expert-indexed form the scales hold one value per expert and the biases
 * n_experts*M values, expert-major (expert e's row r at e*M + r). */
typedef struct {
    const double *up_bias;
    const double *gate_bias;
    const double *up_scale;
    const double *gate_scale;
    int glu_op;
    double limit;      /* SWIGLU_CLAMP */
} orc_epilogue;

/* out[j*M + r] for r < M, j < n. W_gate may be NULL (no gate). */
int orc_mmvq_ex(const uint8_t *W_up, const uint8_t *W_gate, int type,
                int64_t M, int64_t K, const uint8_t *y_q, int64_t n,
                const orc_epilogue *epi, double *out);

/* Expert-indexed form of orc_mmvq_ex, out[(t*top_k + k)*M + r]. With
 * shared_up non-NULL, a shared expert (matrices shared_up / shared_gate,
 * same shape and type) is applied to every token as well:
 * shared_out[t*M + r], with the GLU of epi and no scale or bias. */
int orc_mmvq_id_ex(const uint8_t *W_up, const uint8_t *W_gate,
                   int64_t expert_stride, int n_experts, int type,
                   int64_t M, int64_t K, const uint8_t *y_q,
                   int64_t n_tokens, const int32_t *ids, int top_k,
                   const orc_epilogue *epi, const uint8_t *shared_up,
                   const uint8_t *shared_gate, double *shared_out,
                   double *out);

/* Dequantize one row of K weights to fp64 (w[e] = the weight value of
 * element e), and one column of q8_1 to fp64 (y[e] = d * q[e]). */
int orc_dequantize_row(int type, const uint8_t *row, int64_t K, double *w);
int orc_dequantize_q8_1(const uint8_t *y_q, int64_t K, double *y);

/* The 6-bit scale and min of Q4_K sub-block t (0..7) from the 12 packed
 * scale bytes. */
void orc_q4_k_scale_min(const uint8_t *scales, int t, int *sc, int *m);

#ifdef __cplusplus
}
#endif

#endif
