// kernels_mmq.hip - launches of the many-column (MFMA) kernel.
#include "launch.hpp"
#include "mmq_kernel.hpp"

namespace qmv {

// Tiles per workgroup: 2 row tiles x 2 column tiles (32 x 32 outputs), four
// waves splitting K.
int launch_mmq_q4k(const MmqArgs& a, hipStream_t st) {
  constexpr int RT = 2, CT = 2;
  const int64_t gx = (a.M + 16 * RT - 1) / (16 * RT);
  const int64_t gy = (a.n + 16 * CT - 1) / (16 * CT);
  hipLaunchKernelGGL((mmq_q4k_kernel<RT, CT>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(kMmqWaves * kWave), 0, st, a);
  return check_launch();
}

}  // namespace qmv
