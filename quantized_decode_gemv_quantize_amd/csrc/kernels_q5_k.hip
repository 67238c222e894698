// kernels_q5_k.hip - instantiates the MMVQ kernels for the Q5_K format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q5_k() {
  static const Dispatch d = make_dispatch<Q5K, false>();
  return d;
}

}  // namespace qmv
