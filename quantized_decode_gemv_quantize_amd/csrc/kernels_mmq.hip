// kernels_mmq.hip - the many-column (MFMA) kernel on q8_1 columns.
#include "mmq_launch.hpp"

namespace qmv {

int launch_mmq(int type, const MmqArgs& a, hipStream_t st) { return launch_mmq_form<false>(type, a, st); }

}  // namespace qmv
