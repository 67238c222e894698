// kernels_q5_1.hip - instantiates the MMVQ kernels for the Q5_1 format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q5_1() {
  static const Dispatch d = make_dispatch<Q51, false>();
  return d;
}

}  // namespace qmv
