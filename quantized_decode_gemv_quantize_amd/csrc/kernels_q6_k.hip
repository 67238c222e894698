// kernels_q6_k.hip - instantiates the MMVQ kernels for the Q6_K format.
#include "launch.hpp"

namespace qmv {

const Dispatch& dispatch_q6_k() {
  static const Dispatch d = make_dispatch<Q6K, false>();
  return d;
}

}  // namespace qmv
