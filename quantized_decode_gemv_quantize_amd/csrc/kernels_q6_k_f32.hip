// kernels_q6_k_f32.hip - instantiates the MMVQ kernels for the Q6_K format with
// fp32 activations quantized to q8_1 in the kernel prologue.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q6_k_f32() {
  static const Dispatch d = make_dispatch<Q6K, true>();
  return d;
}

}  // namespace qmv
