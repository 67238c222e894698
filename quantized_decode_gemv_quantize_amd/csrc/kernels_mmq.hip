// kernels_mmq.hip - launches of the many-column (MFMA) kernel.
#include <cstdlib>

#include "launch.hpp"
#include "mmq_kernel.hpp"

namespace qmv {

namespace {

template <int RT, int CT, int NW>
int launch_tile(const MmqArgs& a, hipStream_t st) {
  if constexpr (!mmq_fits<RT, CT, NW>()) {
    return MMVQ_ERR_SHAPE;
  } else {
  const int64_t gx = (a.M + 16 * RT - 1) / (16 * RT);
  const int64_t gy = (a.n + 16 * CT - 1) / (16 * CT);
  hipLaunchKernelGGL((mmq_q4k_kernel<RT, CT, NW>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(NW * kWave), 0, st, a);
  return check_launch();
  }
}

int64_t groups(const MmqArgs& a, int rt, int ct) {
  return ((a.M + 16 * rt - 1) / (16 * rt)) * ((a.n + 16 * ct - 1) / (16 * ct));
}

template <int NW>
int launch_waves(const MmqArgs& a, int rt, int ct, hipStream_t st) {
  switch (rt * 10 + ct) {
    case 22: return launch_tile<2, 2, NW>(a, st);
    case 21: return launch_tile<2, 1, NW>(a, st);
    case 11: return launch_tile<1, 1, NW>(a, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

}  // namespace

// Tile (row tiles x column tiles of 16 per workgroup): the largest tile that
// still gives every compute unit a workgroup (larger tiles re-read fewer
// weights and activations) and has no more column tiles than n needs, else
// one tile. When the grid is no larger than the chip, eight waves split K
// instead of four, so each compute unit has more loads in flight.
int launch_mmq_q4k(const MmqArgs& a, hipStream_t st) {
  static const int kTiles[][2] = {{2, 2}, {2, 1}, {1, 1}};
  const int64_t cus = device_cus();
  const int ct_max = (a.n + 15) / 16;
  int rt = 1, ct = 1;
  for (const auto& t : kTiles) {
    if (t[1] <= ct_max && groups(a, t[0], t[1]) >= cus) {
      rt = t[0];
      ct = t[1];
      break;
    }
  }
  int nw = groups(a, rt, ct) <= cus ? 8 : 4;
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_MMQ_TILE")) {
    rt = e[0] - '0';
    ct = e[2] - '0';
  }
  if (const char* e = getenv("MMVQ_MMQ_WAVES")) nw = atoi(e);
#endif
  switch (nw) {
    case 4: return launch_waves<4>(a, rt, ct, st);
    case 8: return launch_waves<8>(a, rt, ct, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

}  // namespace qmv
