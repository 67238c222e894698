// kernels_q4_1.hip - instantiates the MMVQ kernels for the Q4_1 format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q4_1() {
  static const Dispatch d = make_dispatch<Q41, false>();
  return d;
}

}  // namespace qmv
