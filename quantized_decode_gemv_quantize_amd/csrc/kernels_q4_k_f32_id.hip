// kernels_q4_k_f32_id.hip - instantiates the expert-indexed MMVQ kernels for the Q4_K format
// (whole-chunk lane layout) with fp32 activations quantized to q8_1 in the kernel prologue.
#include "launch.hpp"

namespace qmv {

int launch_id_q4k_f32(const RowArgs& a, int64_t K, int n_experts, hipStream_t st) {
  return launch_id<Q4K2, true, 1>(a, K, n_experts, st);
}

int launch_id_glu_q4k_f32(const RowArgs& a, int64_t K, int n_experts, hipStream_t st) {
  return launch_id<Q4K2, true, 2>(a, K, n_experts, st);
}

}  // namespace qmv
