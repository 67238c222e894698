// kernels_q4_k_f32.hip - instantiates the MMVQ kernels for the Q4_K format with
// fp32 activations quantized to q8_1 in the kernel prologue.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q4_k_f32() {
  static const Dispatch d = make_dispatch_q4k<true>();
  return d;
}

}  // namespace qmv
