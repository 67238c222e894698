// api.hip - the C ABI declared in include/mmvq.h.
//
// Every entry point validates its arguments on the host and enqueues
// nothing when they are invalid; it never synchronizes and never aborts.
#include <stdint.h>

#include "../../include/mmvq.h"
#include "launch.hpp"

using namespace qmv;

namespace {

const Dispatch* dispatch_for(int type, bool f32) {
  switch (type) {
    case MMVQ_Q4_0: return f32 ? &dispatch_q4_0_f32() : &dispatch_q4_0();
    case MMVQ_Q4_K: return f32 ? &dispatch_q4_k_f32() : &dispatch_q4_k();
    case MMVQ_Q6_K: return f32 ? &dispatch_q6_k_f32() : &dispatch_q6_k();
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
  if (K / (*d)->qk * (*d)->units_per_block > kLaunchBound) return MMVQ_ERR_SHAPE;
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

int gemv_common(const void* W, int type, int64_t M, int64_t K, const ActIn& in, int64_t n, float* out,
                void* stream) {
  const Dispatch* d;
  RowArgs a;
  const int rc = check_gemv(W, type, M, K, in, n, out, &d, &a);
  if (rc) return rc;
  return d->rows(a, K, n, static_cast<hipStream_t>(stream));
}

int glu_common(const void* W_gate, const void* W_up, int type, int64_t M, int64_t K, const ActIn& in, int64_t n,
               int glu_op, float* out, void* stream) {
  if (!W_gate) return MMVQ_ERR_NULL;
  const Dispatch* d;
  RowArgs a;
  const int rc = check_gemv(W_up, type, M, K, in, n, out, &d, &a);
  if (rc) return rc;
  if (glu_op != MMVQ_GLU_PLAIN && glu_op != MMVQ_GLU_SWIGLU) return MMVQ_ERR_TYPE;
  if (!aligned(W_gate, 16)) return MMVQ_ERR_ALIGN;
  a.Wg = static_cast<const uint8_t*>(W_gate);
  a.glu_op = glu_op;
  return d->rows_glu(a, K, n, static_cast<hipStream_t>(stream));
}

int id_common(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
              int64_t M, int64_t K, const ActIn& in, int64_t n_tokens, const int32_t* ids, int top_k, int glu_op,
              bool fused, float* out, void* stream) {
  if (!ids || (fused && !W_gate)) return MMVQ_ERR_NULL;
  const Dispatch* d;
  RowArgs a;
  const int rc = check_gemv(W_up, type, M, K, in, n_tokens, out, &d, &a);
  if (rc) return rc;
  if (fused && glu_op != MMVQ_GLU_PLAIN && glu_op != MMVQ_GLU_SWIGLU) return MMVQ_ERR_TYPE;
  if (n_experts < 1 || n_experts > 65535 || top_k < 1 || top_k > n_experts || top_k > 64) return MMVQ_ERR_SHAPE;
  if (expert_stride_bytes < M * a.row_bytes) return MMVQ_ERR_SHAPE;
  if (expert_stride_bytes % 16 != 0 || !aligned(ids, 4) || (fused && !aligned(W_gate, 16))) return MMVQ_ERR_ALIGN;
  a.Wg = static_cast<const uint8_t*>(W_gate);
  a.ids = ids;
  a.expert_stride = expert_stride_bytes;
  a.n_tokens = static_cast<int>(n_tokens);
  a.top_k = top_k;
  a.glu_op = glu_op;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return fused ? d->id_glu(a, K, n_experts, st) : d->id(a, K, n_experts, st);
}

ActIn q8(const void* y_q) { return ActIn{y_q, nullptr, 0}; }
ActIn f32(const float* x, int64_t ldx) { return ActIn{nullptr, x, ldx}; }   // x checked non-NULL first

}  // namespace

extern "C" {

int mmvq_type_info(int type, int* block_elems, int* block_bytes) {
  int e, b;
  switch (type) {
    case MMVQ_Q4_0: e = 32; b = 18; break;
    case MMVQ_Q4_K: e = 256; b = 144; break;
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
  if (K < 32 || K % 32 != 0 || n < 1 || n > MMVQ_MAX_COLS || ldx < K) return MMVQ_ERR_SHAPE;
  if (K > (int64_t(1) << 30)) return MMVQ_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(y_q, 16)) return MMVQ_ERR_ALIGN;
  return launch_quantize_q8_1(x, static_cast<uint8_t*>(y_q), K, n, ldx, static_cast<hipStream_t>(stream));
}

int mmvq(const void* W, int type, int64_t M, int64_t K, const void* y_q, int64_t n, float* out, void* stream) {
  return gemv_common(W, type, M, K, q8(y_q), n, out, stream);
}

int mmvq_glu(const void* W_gate, const void* W_up, int type, int64_t M, int64_t K, const void* y_q, int64_t n,
             int glu_op, float* out, void* stream) {
  return glu_common(W_gate, W_up, type, M, K, q8(y_q), n, glu_op, out, stream);
}

int mmvq_id(const void* W, int64_t expert_stride_bytes, int n_experts, int type, int64_t M, int64_t K,
            const void* y_q, int64_t n_tokens, const int32_t* ids, int top_k, float* out, void* stream) {
  return id_common(nullptr, W, expert_stride_bytes, n_experts, type, M, K, q8(y_q), n_tokens, ids, top_k, 0,
                   false, out, stream);
}

int mmvq_id_glu(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
                int64_t M, int64_t K, const void* y_q, int64_t n_tokens, const int32_t* ids, int top_k,
                int glu_op, float* out, void* stream) {
  return id_common(W_gate, W_up, expert_stride_bytes, n_experts, type, M, K, q8(y_q), n_tokens, ids, top_k,
                   glu_op, true, out, stream);
}

int mmvq_f32(const void* W, int type, int64_t M, int64_t K, const float* x, int64_t n, int64_t ldx, float* out,
             void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return gemv_common(W, type, M, K, f32(x, ldx), n, out, stream);
}

int mmvq_glu_f32(const void* W_gate, const void* W_up, int type, int64_t M, int64_t K, const float* x, int64_t n,
                 int64_t ldx, int glu_op, float* out, void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return glu_common(W_gate, W_up, type, M, K, f32(x, ldx), n, glu_op, out, stream);
}

int mmvq_id_f32(const void* W, int64_t expert_stride_bytes, int n_experts, int type, int64_t M, int64_t K,
                const float* x, int64_t n_tokens, int64_t ldx, const int32_t* ids, int top_k, float* out,
                void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return id_common(nullptr, W, expert_stride_bytes, n_experts, type, M, K, f32(x, ldx), n_tokens, ids, top_k, 0,
                   false, out, stream);
}

int mmvq_id_glu_f32(const void* W_gate, const void* W_up, int64_t expert_stride_bytes, int n_experts, int type,
                    int64_t M, int64_t K, const float* x, int64_t n_tokens, int64_t ldx, const int32_t* ids,
                    int top_k, int glu_op, float* out, void* stream) {
  if (!x) return MMVQ_ERR_NULL;
  return id_common(W_gate, W_up, expert_stride_bytes, n_experts, type, M, K, f32(x, ldx), n_tokens, ids, top_k,
                   glu_op, true, out, stream);
}

int mmvq_block_dots(const void* W, int type, int64_t M, int64_t K, const void* y_q, int64_t n, int32_t* dots,
                    void* stream) {
  const Dispatch* d;
  RowArgs a;
  const int rc = check_gemv(W, type, M, K, q8(y_q), n, reinterpret_cast<const float*>(dots), &d, &a);
  if (rc) return rc;
  return d->block_dots(a.W, a.y, dots, M, K, n, static_cast<hipStream_t>(stream));
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
