// kernels_q4_k.hip - instantiates the MMVQ kernels for the Q4_K format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q4_k() {
  static const Dispatch d = make_dispatch_q4k<false>();
  return d;
}

}  // namespace qmv
