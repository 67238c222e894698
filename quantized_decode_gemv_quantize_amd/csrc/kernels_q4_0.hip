// kernels_q4_0.hip - instantiates the MMVQ kernels for the Q4_0 format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q4_0() {
  static const Dispatch d = make_dispatch<Q40, false>();
  return d;
}

}  // namespace qmv
