// kernels_q5_0.hip - instantiates the MMVQ kernels for the Q5_0 format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q5_0() {
  static const Dispatch d = make_dispatch<Q50, false>();
  return d;
}

}  // namespace qmv
