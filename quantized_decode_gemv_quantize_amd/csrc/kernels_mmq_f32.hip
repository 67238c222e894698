// kernels_mmq_f32.hip - the many-column (MFMA) kernel on fp32 columns, each
// staged block quantized to q8_1 in the kernel.
#include "mmq_launch.hpp"

namespace qmv {

int launch_mmq_f32(int type, const MmqArgs& a, hipStream_t st) { return launch_mmq_form<true>(type, a, st); }

}  // namespace qmv
