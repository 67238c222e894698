// api.hip - the C ABI declared in include/mmvq.h.
//
// Every entry point validates its arguments on the host and enqueues
// nothing when they are invalid; it never synchronizes and never aborts.
#include <cstdlib>
#include <stdint.h>

#include "../../include/mmvq.h"
#include "launch.hpp"
#include "mmq_plan.hpp"

using namespace qmv;

namespace {

const Dispatch* dispatch_for(int type, bool f32) {
  switch (type) {
    case MMVQ_Q4_0: return f32 ? &dispatch_q4_0_f32() : &dispatch_q4_0();
    case MMVQ_Q8_0: return f32 ? &dispatch_q8_0_f32() : &dispatch_q8_0();
    case MMVQ_Q4_K: return f32 ? &dispatch_q4_k_f32() : &dispatch_q4_k();
    case MMVQ_Q6_K: return f32 ? &dispatch_q6_k_f32() : &dispatch_q6_k();
    case MMVQ_Q4_1: return f32 ? &dispatch_q4_1_f32() : &dispatch_q4_1();
    case MMVQ_Q5_0: return f32 ? &dispatch_q5_0_f32() : &dispatch_q5_0();
    case MMVQ_Q5_1: return f32 ? &dispatch_q5_1_f32() : &dispatch_q5_1();
    case MMVQ_Q5_K: return f32 ? &dispatch_q5_k_f32() : &dispatch_q5_k();
    default: return nullptr;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Activation operand of a weight-matrix call: q8_1 columns y_q (x NULL), or
// fp32 columns x with column stride ldx, quantized inside the kernel.
struct ActIn {
  const void* y_q;
  const float* x;
  int64_t ldx;
};

// Shared checks of the weight-matrix calls; fills the common RowArgs fields.
int check_gemv(const void* W, int type, int64_t M, int64_t K, const ActIn& in, int64_t n, const float* out,
               const Dispatch** d, RowArgs* a) {
  const bool f32 = in.x != nullptr;
  if (!W || !(f32 || in.y_q) || !out) return MMVQ_ERR_NULL;
  *d = dispatch_for(type, f32);
  if (!*d) return MMVQ_ERR_TYPE;
  if (M < 1 || K < 1 || K % (*d)->qk != 0 || n < 1 || n > MMVQ_MAX_COLS) return MMVQ_ERR_SHAPE;
  if (K / (*d)->qk * (*d)->units_per_block > kMaxUnitsPerRow) return MMVQ_ERR_SHAPE;
  if (M > (int64_t(1) << 40) / K) return MMVQ_ERR_SHAPE;
  if (f32 && (in.ldx < K || in.ldx > (int64_t(1) << 40))) return MMVQ_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(out, 4)) return MMVQ_ERR_ALIGN;
  if (f32 ? !aligned(in.x, 4) : !aligned(in.y_q, 16)) return MMVQ_ERR_ALIGN;
  *a = RowArgs{};
  a->W = static_cast<const uint8_t*>(W);
  a->y = static_cast<const uint8_t*>(in.y_q);
  a->x = in.x;
  a->ldx = in.ldx;
  a->out = const_cast<float*>(out);
  a->M = M;
  a->row_bytes = K / (*d)->qk * (*d)->block_bytes;
  a->ycol_bytes = K / 32 * kQ8Bytes;
  return MMVQ_OK;
}

bool valid_glu(int op) { return op >= MMVQ_GLU_PLAIN && op <= MMVQ_GLU_SWIGLU_CLAMP; }

// The GLU-only calls (no epilogue struct) take the ops without a caller
// parameter; SWIGLU_CLAMP needs the limit that only mmvq_ex carries.
int glu_only_op(int op) { return valid_glu(op) && op != MMVQ_GLU_SWIGLU_CLAMP ? MMVQ_OK : MMVQ_ERR_TYPE; }

// Epilogue fields of RowArgs from a caller's (host) mmvq_epilogue.
int set_epilogue(const mmvq_epilogue* epi, bool gate, RowArgs* a) {
  if (!epi) return MMVQ_OK;
  const float* ptrs[4] = {epi->up_bias, epi->gate_bias, epi->up_scale, epi->gate_scale};
  for (const float* q : ptrs)
    if (q && !aligned(q, 4)) return MMVQ_ERR_ALIGN;
  if (gate && !valid_glu(epi->glu_op)) return MMVQ_ERR_TYPE;
  a->up_bias = epi->up_bias;
  a->up_scale = epi->up_scale;
  a->gate_bias = gate ? epi->gate_bias : nullptr;
  a->gate_scale = gate ? epi->gate_scale : nullptr;
  a->glu_op = epi->glu_op;
  a->glu_limit = epi->glu_limit;
  return MMVQ_OK;
}

// The activation operand of the _ex calls: exactly one of y_q and x.
int act_in(const void* y_q, const float* x, int64_t ldx, ActIn* in) {
  if (!y_q && !x) return MMVQ_ERR_NULL;
  if (y_q && x) return MMVQ_ERR_SHAPE;
  *in = ActIn{y_q, x, ldx};
  return MMVQ_OK;
}

ActIn q8(const void* y_q) { return ActIn{y_q, nullptr, 0}; }
ActIn f32(const float* x, int64_t ldx) { return ActIn{nullptr, x, ldx}; }   // x checked non-NULL first

mmvq_epilogue glu_only(int glu_op) {
  mmvq_epilogue e{};
  e.glu_op = glu_op;
  return e;
}

// Formats the matrix-core kernel takes: all of them (the forms it does not
// take run more than MMVQ_MAX_COLS columns as column groups through the row
// kernels).
bool mmq_type(int type) {
  return type == MMVQ_Q4_K || type == MMVQ_Q6_K || type == MMVQ_Q4_0 || type == MMVQ_Q8_0 || type == MMVQ_Q4_1 ||
         type == MMVQ_Q5_0 || type == MMVQ_Q5_1 || type == MMVQ_Q5_K;
}

// Many columns (up to MMVQ_MAX_COLS_BATCH): the MFMA kernel, q8_1 or fp32
// activations (the fp32 form quantizes its staged blocks in the kernel, to
// the same codes), K a multiple of 256, with or without a gate (W_gate
// NULL); the whole epilogue applies.
int mmq_common(const void* W, const void* W_gate, int type, int64_t M, int64_t K, const ActIn& in, int64_t n,
               const mmvq_epilogue* epi, float* out, void* stream) {
  const bool f32 = in.x != nullptr;
  if (!W || !(f32 || in.y_q) || !out) return MMVQ_ERR_NULL;
  const Dispatch* d = dispatch_for(type, false);
  if (!d) return MMVQ_ERR_TYPE;
  if (!mmq_type(type)) return MMVQ_ERR_TYPE;
  if (M < 1 || K < 1 || K % 256 != 0 || n < 1 || n > MMVQ_MAX_COLS_BATCH) return MMVQ_ERR_SHAPE;
  if (M > (int64_t(1) << 40) / K || K / 256 > (int64_t(1) << 24)) return MMVQ_ERR_SHAPE;
  if (f32 && (in.ldx < K || in.ldx > (int64_t(1) << 40))) return MMVQ_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(out, 4)) return MMVQ_ERR_ALIGN;
  if (f32 ? !aligned(in.x, 4) : !aligned(in.y_q, 16)) return MMVQ_ERR_ALIGN;
  if (W_gate && !aligned(W_gate, 16)) return MMVQ_ERR_ALIGN;
  RowArgs ra{};
  int rc = set_epilogue(epi, W_gate != nullptr, &ra);
  if (rc) return rc;
  MmqArgs a{};
  a.W = static_cast<const uint8_t*>(W);
  a.Wg = static_cast<const uint8_t*>(W_gate);
  a.y = static_cast<const uint8_t*>(in.y_q);
  a.x = in.x;
  a.ldx = in.ldx;
  a.out = out;
  a.up_bias = ra.up_bias;
  a.up_scale = ra.up_scale;
  a.gate_bias = ra.gate_bias;
  a.gate_scale = ra.gate_scale;
  a.glu_op = ra.glu_op;
  a.glu_limit = ra.glu_limit;
  a.M = M;
  a.row_bytes = K / d->qk * d->block_bytes;
  a.ycol_bytes = K / 32 * kQ8Bytes;
  a.n = static_cast<int>(n);
  a.nsb = static_cast<int>(K / 256);
  return f32 ? launch_mmq_f32(type, a, static_cast<hipStream_t>(stream))
             : launch_mmq(type, a, static_cast<hipStream_t>(stream));
}

// Columns from which the matrix-core kernel takes a q8_1 product (K a
// multiple of 256): where it measured faster than the row kernels at
// 4096x14336 and 14336x4096 (us, row kernels / matrix cores). Without a
// gate: Q5_K from 5 (24.6 / 16.3 and 19.6 / 16.5 at n = 5), Q4_K from 6
// (one 16-column tile: ~14.5 us for any n <= 16), Q6_K from 7 (57.7 / 31.5
// and 42.8 / 29.0 at n = 7), Q4_0, Q5_0 and Q8_0 from 8 (22.0 / 18.4 and
// 19.1 / 19.5 for Q8_0 at n = 8), Q4_1 and Q5_1 never below 9. Gate/up at
// 14336x4096: Q5_K from 5 (33.4 / 29.5), Q4_K from 7 (28.5 / 25.4; 24.8 /
// 25.3 at 6), the others from 9 (Q6_K 75.3 / 75.7 at 8). 0: not a type.
int mmq_min_cols(int type, bool gate) {
  switch (type) {
    case MMVQ_Q5_K: return 5;
    case MMVQ_Q4_K: return gate ? 7 : 6;
    case MMVQ_Q6_K: return gate ? MMVQ_MAX_COLS + 1 : 7;
    case MMVQ_Q4_0:
    case MMVQ_Q5_0:
    case MMVQ_Q8_0: return gate ? MMVQ_MAX_COLS + 1 : 8;
    case MMVQ_Q4_1:
    case MMVQ_Q5_1: return MMVQ_MAX_COLS + 1;
    default: return 0;
  }
}

// The same for fp32 activations, where the matrix-core kernel quantizes its
// columns again in every row-tile workgroup (about 35 us at these shapes
// for any n <= 16) and the row kernels quantize in their prologue: measured
// at 4096x14336 without a gate and 14336x4096 with one (us, row kernels /
// matrix cores). Without a gate Q6_K from 6 (45.2 / 42.6; 159 / 43 at 7),
// Q5_K from 8 (36.6 / 36.3), the others never below 9 (Q4_K 25.3 / 38.2 at
// 8). With a gate, where the row kernels hold the raw columns of two weight
// streams: Q4_0, Q5_0 and Q5_K from 4 (Q5_K 50.6 / 39.4), the others from 5
// (Q4_K 50.1 / 35.0; 33.3 / 35.6 at 4). 0: not a type.
int mmq_min_cols_f32(int type, bool gate) {
  switch (type) {
    case MMVQ_Q4_0:
    case MMVQ_Q5_0: return gate ? 4 : MMVQ_MAX_COLS + 1;
    case MMVQ_Q5_K: return gate ? 4 : 8;
    case MMVQ_Q6_K: return gate ? 5 : 6;
    case MMVQ_Q4_K:
    case MMVQ_Q8_0:
    case MMVQ_Q4_1:
    case MMVQ_Q5_1: return gate ? 5 : MMVQ_MAX_COLS + 1;
    default: return 0;
  }
}

// Plain or gate/up product with an optional epilogue (W_gate NULL: no gate).
// More than MMVQ_MAX_COLS columns outside the matrix-core kernel's forms
// (K not a multiple of 256) run as groups of at most
// MMVQ_MAX_COLS columns through the row kernels, each group reading the
// weights again; all arguments are checked before the first group is
// enqueued.
int rows_common(const void* W_up, const void* W_gate, int type, int64_t M, int64_t K, const ActIn& in, int64_t n,
                const mmvq_epilogue* epi, float* out, void* stream) {
  const bool mmq_form = K % 256 == 0 && mmq_type(type);
  const int mmq_from = in.x ? mmq_min_cols_f32(type, W_gate != nullptr) : mmq_min_cols(type, W_gate != nullptr);
  if (mmq_form && n >= mmq_from) return mmq_common(W_up, W_gate, type, M, K, in, n, epi, out, stream);
#ifdef QMV_TUNING
  if (getenv("MMVQ_FORCE_MMQ") && mmq_form) return mmq_common(W_up, W_gate, type, M, K, in, n, epi, out, stream);
#endif
  if (n > MMVQ_MAX_COLS_BATCH) return MMVQ_ERR_SHAPE;
  const int64_t n0 = n < MMVQ_MAX_COLS ? n : MMVQ_MAX_COLS;
  const Dispatch* d;
  RowArgs a;
  int rc = check_gemv(W_up, type, M, K, in, n0, out, &d, &a);
  if (rc) return rc;
  if (W_gate && !aligned(W_gate, 16)) return MMVQ_ERR_ALIGN;
  rc = set_epilogue(epi, W_gate != nullptr, &a);
  if (rc) return rc;
  a.Wg = static_cast<const uint8_t*>(W_gate);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // column groups: the activation columns and outputs of group g start
  // g*MMVQ_MAX_COLS columns in (the row kernels need 4-byte aligned q8_1
  // columns, which every column of a 16-byte aligned y_q is)
  for (int64_t j0 = 0; j0 < n; j0 += MMVQ_MAX_COLS) {
    const int64_t nn = n - j0 < MMVQ_MAX_COLS ? n - j0 : MMVQ_MAX_COLS;
    RowArgs g = a;
    if (in.x) g.x = a.x + j0 * a.ldx;
    else g.y = a.y + j0 * a.ycol_bytes;
    g.out = a.out + j0 * M;
    rc = W_gate ? d->rows_glu(g, K, nn, st) : d->rows(g, K, nn, st);
    if (rc) return rc;
  }
  return MMVQ_OK;
}

// Expert-indexed product with an optional epilogue and shared expert.
int id_common(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
              int64_t M, int64_t K, const ActIn& in, int64_t n_tokens, const int32_t* ids, int top_k,
              const mmvq_epilogue* epi, const void* shared_up, const void* shared_gate, float* shared_out,
              float* out, void* stream) {
  if (!ids) return MMVQ_ERR_NULL;
  if (shared_up && (!shared_out || (W_gate && !shared_gate))) return MMVQ_ERR_NULL;
  const Dispatch* d;
  RowArgs a;
  int rc = check_gemv(W_up, type, M, K, in, n_tokens, out, &d, &a);
  if (rc) return rc;
  const int slices = n_experts + (shared_up ? 1 : 0);
  if (n_experts < 1 || slices > 65535 || top_k < 1 || top_k > n_experts || top_k > 64) return MMVQ_ERR_SHAPE;
  if (expert_stride_bytes < M * a.row_bytes) return MMVQ_ERR_SHAPE;
  if (expert_stride_bytes % 16 != 0 || !aligned(ids, 4) || (W_gate && !aligned(W_gate, 16))) return MMVQ_ERR_ALIGN;
  if (shared_up && (!aligned(shared_up, 16) || (W_gate && !aligned(shared_gate, 16)) || !aligned(shared_out, 4)))
    return MMVQ_ERR_ALIGN;
  rc = set_epilogue(epi, W_gate != nullptr, &a);
  if (rc) return rc;
  a.Wg = static_cast<const uint8_t*>(W_gate);
  a.ids = ids;
  a.expert_stride = expert_stride_bytes;
  a.n_tokens = static_cast<int>(n_tokens);
  a.top_k = top_k;
  a.n_experts = n_experts;
  a.Ws_up = static_cast<const uint8_t*>(shared_up);
  a.Ws_gate = W_gate ? static_cast<const uint8_t*>(shared_gate) : nullptr;
  a.shared_out = shared_up ? shared_out : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return W_gate ? d->id_glu(a, K, n_experts, st) : d->id(a, K, n_experts, st);
}

}  // namespace

extern "C" {

int mmvq_many_columns_min(int type, int gated, int fp32, int* n_min) {
  if (!n_min) return MMVQ_ERR_NULL;
  const int m = fp32 ? mmq_min_cols_f32(type, gated != 0) : mmq_min_cols(type, gated != 0);
  if (m == 0) return MMVQ_ERR_TYPE;
  *n_min = m;
  return MMVQ_OK;
}

int mmvq_type_info(int type, int* block_elems, int* block_bytes) {
  int e, b;
  switch (type) {
    case MMVQ_Q4_0: e = 32; b = 18; break;
    case MMVQ_Q4_1: e = 32; b = 20; break;
    case MMVQ_Q5_0: e = 32; b = 22; break;
    case MMVQ_Q5_1: e = 32; b = 24; break;
    case MMVQ_Q8_0: e = 32; b = 34; break;
    case MMVQ_Q4_K: e = 256; b = 144; break;
    case MMVQ_Q5_K: e = 256; b = 176; break;
    case MMVQ_Q6_K: e = 256; b = 210; break;
    case MMVQ_Q8_1: e = 32; b = 36; break;
    default: return MMVQ_ERR_TYPE;
  }
  if (block_elems) *block_elems = e;
  if (block_bytes) *block_bytes = b;
  return MMVQ_OK;
}

int mmvq_quantize_q8_1(const float* x, int64_t K, int64_t n, int64_t ldx, void* y_q, void* stream) {
  if (!x || !y_q) return MMVQ_ERR_NULL;
  if (K < 32 || K % 32 != 0 || n < 1 || n > MMVQ_MAX_COLS_BATCH || ldx < K) return MMVQ_ERR_SHAPE;
  if (K > (int64_t(1) << 30)) return MMVQ_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(y_q, 16)) return MMVQ_ERR_ALIGN;
  return launch_quantize_q8_1(x, static_cast<uint8_t*>(y_q), K, n, ldx, static_cast<hipStream_t>(stream));
}

int mmvq(const void* W, int type, int64_t M, int64_t K, const void* y_q, int64_t n, float* out, void* stream) {
  return rows_common(W, nullptr, type, M, K, q8(y_q), n, nullptr, out, stream);
}

int mmvq_glu(const void* W_gate, const void* W_up, int type, int64_t M, int64_t K, const void* y_q, int64_t n,
             int glu_op, float* out, void* stream) {
  if (!W_gate) return MMVQ_ERR_NULL;
  if (glu_only_op(glu_op)) return MMVQ_ERR_TYPE;
  const mmvq_epilogue e = glu_only(glu_op);
  return rows_common(W_up, W_gate, type, M, K, q8(y_q), n, &e, out, stream);
}

int mmvq_id(const void* W, int64_t expert_stride_bytes, int n_experts, int type, int64_t M, int64_t K,
            const void* y_q, int64_t n_tokens, const int32_t* ids, int top_k, float* out, void* stream) {
  return id_common(nullptr, W, expert_stride_bytes, n_experts, type, M, K, q8(y_q), n_tokens, ids, top_k, nullptr,
                   nullptr, nullptr, nullptr, out, stream);
}

int mmvq_id_glu(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
                int64_t M, int64_t K, const void* y_q, int64_t n_tokens, const int32_t* ids, int top_k,
                int glu_op, float* out, void* stream) {
  if (!W_gate) return MMVQ_ERR_NULL;
  if (glu_only_op(glu_op)) return MMVQ_ERR_TYPE;
  const mmvq_epilogue e = glu_only(glu_op);
  return id_common(W_gate, W_up, expert_stride_bytes, n_experts, type, M, K, q8(y_q), n_tokens, ids, top_k, &e,
                   nullptr, nullptr, nullptr, out, stream);
}

int mmvq_f32(const void* W, int type, int64_t M, int64_t K, const float* x, int64_t n, int64_t ldx, float* out,
             void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return rows_common(W, nullptr, type, M, K, f32(x, ldx), n, nullptr, out, stream);
}

int mmvq_glu_f32(const void* W_gate, const void* W_up, int type, int64_t M, int64_t K, const float* x, int64_t n,
                 int64_t ldx, int glu_op, float* out, void* stream) {
  if (!x || !W_gate) return MMVQ_ERR_NULL;
  if (glu_only_op(glu_op)) return MMVQ_ERR_TYPE;
  const mmvq_epilogue e = glu_only(glu_op);
  return rows_common(W_up, W_gate, type, M, K, f32(x, ldx), n, &e, out, stream);
}

int mmvq_id_f32(const void* W, int64_t expert_stride_bytes, int n_experts, int type, int64_t M, int64_t K,
                const float* x, int64_t n_tokens, int64_t ldx, const int32_t* ids, int top_k, float* out,
                void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return id_common(nullptr, W, expert_stride_bytes, n_experts, type, M, K, f32(x, ldx), n_tokens, ids, top_k,
                   nullptr, nullptr, nullptr, nullptr, out, stream);
}

int mmvq_id_glu_f32(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
                    int64_t M, int64_t K, const float* x, int64_t n_tokens, int64_t ldx, const int32_t* ids,
                    int top_k, int glu_op, float* out, void* stream) {
  if (!x || !W_gate) return MMVQ_ERR_NULL;
  if (glu_only_op(glu_op)) return MMVQ_ERR_TYPE;
  const mmvq_epilogue e = glu_only(glu_op);
  return id_common(W_gate, W_up, expert_stride_bytes, n_experts, type, M, K, f32(x, ldx), n_tokens, ids, top_k,
                   &e, nullptr, nullptr, nullptr, out, stream);
}

int mmvq_ex(const void* W_up, const void* W_gate, int type, int64_t M, int64_t K, const void* y_q, const float* x,
            int64_t ldx, int64_t n, const mmvq_epilogue* epi, float* out, void* stream) {
  ActIn in;
  const int rc = act_in(y_q, x, ldx, &in);
  if (rc) return rc;
  return rows_common(W_up, W_gate, type, M, K, in, n, epi, out, stream);
}

int mmvq_id_ex(const void* W_up, const void* W_gate, int64_t expert_stride_bytes, int n_experts, int type,
               int64_t M, int64_t K, const void* y_q, const float* x, int64_t ldx, int64_t n_tokens,
               const int32_t* ids, int top_k, const mmvq_epilogue* epi, const void* shared_up,
               const void* shared_gate, float* shared_out, float* out, void* stream) {
  ActIn in;
  const int rc = act_in(y_q, x, ldx, &in);
  if (rc) return rc;
  return id_common(W_gate, W_up, expert_stride_bytes, n_experts, type, M, K, in, n_tokens, ids, top_k, epi,
                   shared_up, shared_gate, shared_out, out, stream);
}

int mmvq_block_dots(const void* W, int type, int64_t M, int64_t K, const void* y_q, int64_t n, int32_t* dots,
                    void* stream) {
  const Dispatch* d;
  RowArgs a;
  const int rc = check_gemv(W, type, M, K, q8(y_q), n, reinterpret_cast<const float*>(dots), &d, &a);
  if (rc) return rc;
  return d->block_dots(a.W, a.y, dots, M, K, n, static_cast<hipStream_t>(stream));
}

int mmvq_read_probe(const void* src, int64_t bytes, void* sink, void* stream) {
  if (!src || !sink) return MMVQ_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return MMVQ_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return MMVQ_ERR_ALIGN;
  return launch_read_probe(static_cast<const uint8_t*>(src), bytes, static_cast<uint32_t*>(sink),
                           static_cast<hipStream_t>(stream));
}

const char* mmvq_strerror(int code) {
  switch (code) {
    case MMVQ_OK: return "success";
    case MMVQ_ERR_NULL: return "a required pointer is NULL";
    case MMVQ_ERR_TYPE: return "unsupported weight type or glu_op";
    case MMVQ_ERR_SHAPE: return "invalid shape (K not a multiple of the block, n, M, top_k or stride out of range)";
    case MMVQ_ERR_ALIGN: return "pointer or stride not aligned as required";
    case MMVQ_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    default: return "unknown error code";
  }
}

}  // extern "C"
