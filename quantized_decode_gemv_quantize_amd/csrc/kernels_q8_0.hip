// kernels_q8_0.hip - instantiates the MMVQ kernels for the Q8_0 format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q8_0() {
  static const Dispatch d = make_dispatch<Q80, false>();
  return d;
}

}  // namespace qmv
