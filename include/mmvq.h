/*
 * mmvq.h - C ABI of the MI355X (gfx950) decode-time quantized mat-vec.
 *
 * The library computes, on the GPU, the quantized matrix-vector product used
 * at decode time: an fp32 activation is first quantized to q8_1 blocks, then
 * every row of a block-quantized weight matrix (Q4_0, Q4_K or Q6_K) is
 * reduced against it with integer block dot products, the block scales
 * applied afterwards. Variants: n = 1..8 activation columns against one
 * weight read, a fused gate/up GLU epilogue, and an expert-indexed product.
 *
 * Citations (sources of each operation's definition):
 *   [MMVQ §X]   page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时一条量化权重
 *               如何被 dp4a 逐块点积" (pinghaoyang.com.cn), section X.
 *   [GGUF16 §X] page "GGUF 量化内幕：第16章 llama.cpp 量化代码架构"
 *               (cnblogs apachecn), section X.
 *   [LLM §X]    page "解构LLM：以llama.cpp分析模型推理过程" (laumy.tech),
 *               section X.
 *
 * Conventions for every entry point:
 *   - Pointers to data (x, W, y_q, ids, out, dots) are DEVICE pointers. The
 *     caller allocates, owns and frees them; the library keeps no
 *     allocation, no pointer and no mutable global state, and may be called
 *     from several host threads at once.
 *   - `stream` is a hipStream_t (NULL = the null stream). All work is
 *     enqueued asynchronously on it; the library never synchronizes. Inputs
 *     must stay valid and outputs untouched until the stream reaches the
 *     enqueued work.
 *   - Shapes: M output rows, K the reduction length (row length), n
 *     activation columns (1..8).
 *   - Weights W: M rows stored back to back, each K/qk blocks of the type's
 *     block size (qk = 32 for Q4_0, 256 for Q4_K and Q6_K); row stride
 *     (K/qk)*block_bytes. Byte layouts:
 *       Q4_0 (18 B / 32): fp16 d @0, 16 B of 4-bit codes @2; qs[j] low
 *            nibble = element j, high nibble = element j+16; w = d*(q-8).
 *       Q8_0 (34 B / 32): fp16 d @0, 32 int8 codes @2; w = d*q.
 *       Q4_K (144 B / 256): fp16 d @0, fp16 dmin @2, 12 B of packed 6-bit
 *            sub-block scales and mins @4, 128 B of 4-bit codes @16;
 *            w = d*sc*q - dmin*m.
 *       Q6_K (210 B / 256): 128 B low code bits @0, 64 B high code bits
 *            @128, 16 int8 sub-block scales @192, fp16 d @208;
 *            w = d*sc*(q-32).
 *   - Activations y_q: n columns, column j at y_q + j*(K/32)*36 bytes, each
 *     K/32 q8_1 blocks of 36 bytes: fp16 d @0, fp16 s = d*sum(q) @2, 32 int8
 *     codes @4 [MMVQ §激活的量化].
 *   - Output out: fp32, column-major by activation column:
 *     out[j*M + r] is row r against column j [MMVQ §归约与写出].
 *   - Alignment: W and y_q 16-byte aligned, x, out, ids and dots 4-byte
 *     aligned; expert_stride_bytes a multiple of 16.
 *   - Return value: MMVQ_OK (0) or a negative MMVQ_ERR_* code. Arguments are
 *     validated on the host before anything is enqueued; an invalid call
 *     enqueues nothing. No entry point aborts the process.
 *   - Expert ids are not checked on the GPU: an id outside 0..n_experts-1
 *     reads outside the weights and is undefined behaviour.
 */
#ifndef MMVQ_H
#define MMVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Type ids follow the ggml numbering, whose ids are never reused
 * [GGUF16 §16.1.1]. Q4_1, Q5_0, Q5_1 and Q5_K are named on the pages without
 * their layouts (old-style blocks [MMVQ §权重的排法]; Q5_K among the
 * min-term formats [MMVQ §激活的量化]); the layouts taken are the published
 * GGUF block definitions:
 *   Q4_1 20 B / 32: fp16 d, fp16 m, 16 nibble bytes; weight d*q + m
 *   Q5_0 22 B / 32: fp16 d, 4 bytes of fifth bits, 16 nibble bytes;
 *                   weight d*(q - 16)
 *   Q5_1 24 B / 32: fp16 d, fp16 m, 4 bytes of fifth bits, 16 nibble bytes;
 *                   weight d*q + m
 *   Q5_K 176 B / 256: fp16 d, fp16 dmin, the 12 Q4_K scale bytes, 32 bytes
 *                   of fifth bits, 128 nibble bytes; weight d*sc*q - dmin*m
 * (nibbles as Q4_0 / Q4_K; bit e of the 32-bit fifth-bit word is bit 4 of
 * element e; in Q5_K bit t of qh[l] for element l of sub-block t's run).
 * The old-style formats take their offset term from the q8_1 block's s:
 * d*d8*sum(q*qy) + m*s, Q5_0 d*(d8*sum(q*qy) - 16*s). */
enum {
    MMVQ_Q4_0 = 2,
    MMVQ_Q4_1 = 3,
    MMVQ_Q5_0 = 6,
    MMVQ_Q5_1 = 7,
    MMVQ_Q8_0 = 8,
    MMVQ_Q8_1 = 9,
    MMVQ_Q4_K = 12,
    MMVQ_Q5_K = 13,
    MMVQ_Q6_K = 14
};

/* GLU of the fused gate/up variants [MMVQ §融合]. The page's epilogue
 * switch names these ops and calls device functions whose bodies it does
 * not print; the definitions below are this library's readings:
 *   GEGLU: gelu in the tanh form published with GELU (Hendrycks and Gimpel,
 *     2016), gelu(z) = z/2*(1 + tanh(sqrt(2/pi)*(z + 0.044715*z^3)));
 *   SWIGLU_OAI: the clamped SwiGLU published with the gpt-oss models, with
 *     that publication's constants alpha = 1.702 and limit = 7 (the page
 *     calls it with the gate and up values only);
 *   SWIGLU_CLAMP: silu on the same clamps with the caller's limit (the page
 *     passes glu_limit to it).
 * g' = min(gate, limit), u' = clamp(up, -limit, limit). */
enum {
    MMVQ_GLU_PLAIN = 0,        /* out = gate * up                                  */
    MMVQ_GLU_SWIGLU = 1,       /* out = silu(gate) * up, silu(z) = z/(1+e^-z)      */
    MMVQ_GLU_GEGLU = 2,        /* out = gelu(gate) * up, gelu in its tanh form     */
    MMVQ_GLU_SWIGLU_OAI = 3,   /* out = g' * sigmoid(1.702*g') * (u' + 1), limit 7 */
    MMVQ_GLU_SWIGLU_CLAMP = 4  /* out = silu(g') * u', limit = glu_limit           */
};

/* Fused epilogue [MMVQ §融合], applied to each output in the order the
 * pages give: up = up*up_scale + up_bias[r]; with a gate matrix also
 * gate = gate*gate_scale + gate_bias[r], then out = GLU(gate, up); without
 * one, out = up. All pointers are DEVICE pointers (4-byte aligned) or NULL
 * (scale 1, bias 0). In the expert-indexed calls the scales hold one float
 * per expert and the biases n_experts*M floats, expert e's row r at
 * e*M + r. The struct itself is read on the host during the call. */
typedef struct mmvq_epilogue {
    const float *up_bias;
    const float *gate_bias;
    const float *up_scale;
    const float *gate_scale;
    int glu_op;        /* MMVQ_GLU_*, used when a gate matrix is given */
    float glu_limit;   /* SWIGLU_CLAMP                                  */
} mmvq_epilogue;

enum {
    MMVQ_OK = 0,
    MMVQ_ERR_NULL = -1,      /* a required pointer is NULL                         */
    MMVQ_ERR_TYPE = -2,      /* unknown weight type or glu_op                       */
    MMVQ_ERR_SHAPE = -3,     /* K not a multiple of the block, n out of range, row
                                too long, M < 1, ldx < K, top_k outside
                                1..n_experts, ...                                 */
    MMVQ_ERR_ALIGN = -4,     /* a pointer or stride is not aligned as required      */
    MMVQ_ERR_LAUNCH = -5     /* the HIP runtime reported an error at launch         */
};

/* Largest number of activation columns (tokens) per call of the mat-vec
 * forms [MMVQ §分派]. */
#define MMVQ_MAX_COLS 8

/* Largest number of columns of the weight-matrix calls without expert ids
 * (mmvq, mmvq_glu, mmvq_ex and their fp32 forms) and of the quantizer.
 * With K a multiple of 256 these calls run on the matrix cores from
 * mmvq_many_columns_min columns [MMVQ §多个 token 时]; with K not a
 * multiple of 256 they take more than MMVQ_MAX_COLS columns as groups of at
 * most MMVQ_MAX_COLS columns through the row kernels (each group reads the
 * weights again). The expert-indexed calls take at most MMVQ_MAX_COLS
 * tokens. */
#define MMVQ_MAX_COLS_BATCH 256

/* Fewest columns from which mmvq / mmvq_ex (gated = 0) or mmvq_glu /
 * mmvq_ex with a gate matrix (gated != 0), with K a multiple of 256 and
 * q8_1 activations (fp32 = 0) or fp32 activations (fp32 != 0: mmvq_f32,
 * mmvq_glu_f32, mmvq_ex with x), run on the many-column (matrix-core)
 * kernel instead of the row kernels, written to *n_min: the measured
 * crossover of the two on MI355X. q8_1 activations: without a gate Q5_K 5,
 * Q4_K 6, Q6_K 7, Q4_0 / Q5_0 / Q8_0 8, Q4_1 / Q5_1 9; with one Q5_K 5,
 * Q4_K 7, the others 9. fp32 activations (the kernel quantizes its columns
 * in every row-tile workgroup): without a gate Q6_K 6, Q5_K 8, the others
 * 9; with one Q4_0 / Q5_0 / Q5_K 4, the others 5. The two kernels order
 * their sums differently: where a call's fp32 and q8_1 forms run different
 * kernels, they agree within the accumulation-order tolerance, elsewhere
 * bit for bit. Host-only; touches no device. Errors: MMVQ_ERR_NULL (n_min
 * NULL), MMVQ_ERR_TYPE (weight type). */
int mmvq_many_columns_min(int type, int gated, int fp32, int *n_min);

/* Block geometry of a type: elements per block and bytes per block
 * (Q4_0 32/18, Q4_1 32/20, Q5_0 32/22, Q5_1 32/24, Q8_0 32/34, Q4_K 256/144,
 * Q5_K 256/176, Q6_K 256/210, Q8_1 32/36)
 * [MMVQ §一次 vec_dot 的解剖 (format table); GGUF16 §16.1.2, §16.1.3;
 * LLM §量化格式 (Q8_0)].
 * Either output pointer may be NULL. Host-only; touches no device. */
int mmvq_type_info(int type, int *block_elems, int *block_bytes);

/* Quantize n fp32 columns to q8_1 [MMVQ §激活的量化]. Column j of x starts at
 * x + j*ldx (ldx >= K floats); the first K values of each column are used.
 * Per block of 32: d = amax/127 in fp32, q = roundf(x/d) (0 when d == 0),
 * stored fp16(d), fp16(fp32(d*sum(q))), q. y_q receives n*(K/32)*36 bytes.
 * Requires K % 32 == 0, 1 <= n <= MMVQ_MAX_COLS_BATCH. Inputs must be finite; for
 * blocks whose amax is below 127*2^-126 the fp32 d is subnormal and the
 * codes are not meaningful (the computation is still defined). */
int mmvq_quantize_q8_1(const float *x, int64_t K, int64_t n, int64_t ldx,
                       void *y_q, void *stream);

/* out[j*M + r] = sum over the K/qk blocks of row r of W of (block scales)
 * x (integer block dot against column j of y_q), for r < M, j < n
 * [MMVQ §一次 vec_dot 的解剖, §kernel 的形状, §归约与写出, §多个 token 时].
 * Q4_0: d_w*(d8*sum(q*qy) - 8*s) per 32-block. Q8_0: d_w*d8*sum(q*qy)
 * per 32-block. Q4_K: per 32-element
 * sub-block t, d*sc_t*d8*sum(q*qy) - dmin*m_t*d8*sum(qy). Q6_K: per
 * 16-element sub-block, d*sc*d8*sum((q-32)*qy). Accumulated in fp32.
 * Requires K % qk == 0, M >= 1 and 1 <= n <= MMVQ_MAX_COLS_BATCH. A lane
 * of the row kernels (n <= MMVQ_MAX_COLS, and each group of MMVQ_MAX_COLS
 * columns beyond)
 * handles one unit of a row (a block for Q4_0 and Q8_0, half or whole
 * 64-weight chunks for Q4_K, a quarter super-block for Q6_K); rows of more
 * than 512 units are walked by the team in chunks of at most 512 lanes
 * [MMVQ §kernel 的形状: K split across the warps of a block]. Rows of more
 * than 2^24 units (K > 2^29 for Q4_0 and Q8_0, K > 2^30 for Q4_K and Q6_K)
 * and M*K > 2^40 return MMVQ_ERR_SHAPE (the same limits hold for every
 * entry point below except the many-column path).
 * With K a multiple of 256, n >= mmvq_many_columns_min takes the
 * many-column path, where the integer dots of 16 rows x 16 columns x 32
 * elements come from one int8 matrix-core instruction and the same block
 * scales are applied per 32-element block (Q6_K: per 16-element half);
 * K / 256 up to 2^24 there. */
int mmvq(const void *W, int type, int64_t M, int64_t K,
         const void *y_q, int64_t n, float *out, void *stream);

/* Fused gate/up: out[j*M + r] = GLU(g, u) with g the mmvq of W_gate and u
 * the mmvq of W_up (same type and shape), per glu_op: PLAIN, SWIGLU, GEGLU
 * or SWIGLU_OAI (SWIGLU_CLAMP needs a limit: MMVQ_ERR_TYPE here, use
 * mmvq_ex); both weight
 * streams are read in one kernel and the epilogue applies the GLU
 * [MMVQ §融合]. Same requirements as mmvq. */
int mmvq_glu(const void *W_gate, const void *W_up, int type, int64_t M,
             int64_t K, const void *y_q, int64_t n, int glu_op, float *out,
             void *stream);

/* Expert-indexed product (mul_mat_id) [MMVQ §MoE, §正确性上的几个坑].
 * Expert e's M x K matrix starts at W + e*expert_stride_bytes. ids holds
 * n_tokens*top_k int32 expert ids, token-major (device memory). For token
 * t and slot k: out[(t*top_k + k)*M + r] = row r of expert ids[t*top_k+k]
 * against column t of y_q (each token's one q8_1 column serves all its
 * slots). Each expert's weights are read once per call, for all tokens
 * routed to it. Requires 1 <= n_tokens <= MMVQ_MAX_COLS,
 * 1 <= top_k <= n_experts, expert_stride_bytes >= M*row_bytes. */
int mmvq_id(const void *W, int64_t expert_stride_bytes, int n_experts,
            int type, int64_t M, int64_t K, const void *y_q,
            int64_t n_tokens, const int32_t *ids, int top_k, float *out,
            void *stream);

/* Expert-indexed fused gate/up: as mmvq_id with the epilogue of mmvq_glu;
 * W_gate and W_up share expert_stride_bytes. */
int mmvq_id_glu(const void *W_gate, const void *W_up,
                int64_t expert_stride_bytes, int n_experts, int type,
                int64_t M, int64_t K, const void *y_q, int64_t n_tokens,
                const int32_t *ids, int top_k, int glu_op, float *out,
                void *stream);

/* Fused quantize + product, fp32 activations [MMVQ §激活的量化, §融合].
 * The four calls below equal mmvq_quantize_q8_1 followed by mmvq, mmvq_glu,
 * mmvq_id and mmvq_id_glu respectively, bit for bit (except at column
 * counts where only one of the two forms runs the many-column kernel, see
 * mmvq_many_columns_min: there the two agree within the accumulation-order
 * tolerance, the q8_1 codes and scales still identical): each kernel quantizes
 * the slice of x that its lanes multiply, with the quantizer's arithmetic,
 * in registers (the row kernels in their prologue; the many-column kernel
 * each 32-value block it stages, before the block goes to LDS), so the
 * q8_1 columns are never written to memory and one launch replaces two.
 * Column j of x starts at x + j*ldx (ldx >= K floats; the first K values
 * are used; x 4-byte aligned). Each workgroup re-reads its slice of x
 * from cache and quantizes it again; there is no y_q. Same requirements
 * and error codes as the q8_1 forms, plus MMVQ_ERR_SHAPE for ldx < K. */
int mmvq_f32(const void *W, int type, int64_t M, int64_t K, const float *x,
             int64_t n, int64_t ldx, float *out, void *stream);

int mmvq_glu_f32(const void *W_gate, const void *W_up, int type, int64_t M,
                 int64_t K, const float *x, int64_t n, int64_t ldx,
                 int glu_op, float *out, void *stream);

/* Column t of x (x + t*ldx) is token t. */
int mmvq_id_f32(const void *W, int64_t expert_stride_bytes, int n_experts,
                int type, int64_t M, int64_t K, const float *x,
                int64_t n_tokens, int64_t ldx, const int32_t *ids, int top_k,
                float *out, void *stream);

int mmvq_id_glu_f32(const void *W_gate, const void *W_up,
                    int64_t expert_stride_bytes, int n_experts, int type,
                    int64_t M, int64_t K, const float *x, int64_t n_tokens,
                    int64_t ldx, const int32_t *ids, int top_k, int glu_op,
                    float *out, void *stream);

/* General form of mmvq / mmvq_glu / mmvq_f32 / mmvq_glu_f32 with the full
 * epilogue [MMVQ §融合]. W_gate NULL: no gate (out = up after its scale and
 * bias). Activations: exactly one of y_q (q8_1 columns) and x (fp32 columns
 * at stride ldx, quantized in the kernel); neither -> MMVQ_ERR_NULL, both ->
 * MMVQ_ERR_SHAPE. epi NULL: no scale, no bias, and GLU gate*up. Otherwise
 * the requirements and codes of the forms it generalizes. */
int mmvq_ex(const void *W_up, const void *W_gate, int type, int64_t M,
            int64_t K, const void *y_q, const float *x, int64_t ldx,
            int64_t n, const mmvq_epilogue *epi, float *out, void *stream);

/* General form of the expert-indexed calls [MMVQ §MoE, §融合]: routed
 * experts as in mmvq_id / mmvq_id_glu with the epilogue of epi (per-expert
 * scales and bias rows), plus an optional shared expert: with shared_up
 * non-NULL, shared_up (and shared_gate, required when W_gate is given) are
 * M x K matrices of the same type applied to every token, out
 * shared_out[t*M + r] (n_tokens*M floats), with the GLU of epi and no scale
 * or bias; on the GPU it is one more grid slice of the same launch.
 * Requires n_experts + 1 <= 65535 with a shared expert. */
int mmvq_id_ex(const void *W_up, const void *W_gate,
               int64_t expert_stride_bytes, int n_experts, int type,
               int64_t M, int64_t K, const void *y_q, const float *x,
               int64_t ldx, int64_t n_tokens, const int32_t *ids, int top_k,
               const mmvq_epilogue *epi, const void *shared_up,
               const void *shared_gate, float *shared_out, float *out,
               void *stream);

/* TEST SUPPORT: the integer block dots that mmvq forms, through the same
 * device decode routines (for Q4_K, the lane layout the mat-vec takes at
 * that K: half chunks up to K = 16384, whole chunks beyond, the layout of
 * the expert kernels), written instead of being scaled and summed.
 * dots[((j*M + r)*(K/qk) + b)*D + i] with D = 16 for Q4_K (sum(q*qy) of
 * sub-blocks 0..7, then sum(qy) of sub-blocks 0..7), 16 for Q6_K
 * (sum((q-32)*qy) of sub-blocks 0..15), 1 for Q4_0 and Q8_0 (sum(q*qy)).
 * [MMVQ §dp4a, §一次 vec_dot 的解剖]. Same requirements as mmvq. */
int mmvq_block_dots(const void *W, int type, int64_t M, int64_t K,
                    const void *y_q, int64_t n, int32_t *dots, void *stream);

/* MEASUREMENT SUPPORT: reads bytes bytes at src (device, 16-byte aligned,
 * bytes a positive multiple of 16) with 16-byte coalesced loads and does
 * nothing else; sink is a device word it may write (4-byte aligned). The
 * time of this launch is the HBM read ceiling the mat-vec launches are
 * compared with for the same bytes [MMVQ §性能直觉 (decode is bound by the
 * weight read)]. Asynchronous on stream; MMVQ_ERR_* codes as above. */
int mmvq_read_probe(const void *src, int64_t bytes, void *sink, void *stream);

/* Static, human-readable text for a return code. Never NULL. */
const char *mmvq_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MMVQ_H */
