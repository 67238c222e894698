// kernels_q4_1_f32.hip - instantiates the MMVQ kernels for the Q4_1 format with
// fp32 activations quantized to q8_1 in the kernel prologue.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q4_1_f32() {
  static const Dispatch d = make_dispatch<Q41, true>();
  return d;
}

}  // namespace qmv
