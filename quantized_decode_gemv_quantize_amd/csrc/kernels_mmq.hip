// kernels_mmq.hip - launches of the many-column (MFMA) kernel.
#include <cstdlib>

#include "launch.hpp"
#include "mmq_kernel.hpp"

namespace qmv {

namespace {

int64_t groups(const MmqArgs& a, int rt, int ct) {
  return ((a.M + 16 * rt - 1) / (16 * rt)) * ((a.n + 16 * ct - 1) / (16 * ct));
}

// Tiles of the gate/up form: every tile whose two accumulator sets and
// staging buffers fit the registers without spilling.
template <class F, int RT, int CT>
constexpr bool mmq_glu_tile() { return true; }

template <class F, int RT, int CT, int NW, int G>
constexpr bool tile_ok() { return mmq_fits<F, RT, CT, NW, G>() && (G == 1 || mmq_glu_tile<F, RT, CT>()); }

template <class F, int RT, int CT, int NW, int G>
int launch_tile(MmqArgs a, hipStream_t st) {
  if constexpr (!tile_ok<F, RT, CT, NW, G>()) {
    return MMVQ_ERR_SHAPE;
  } else {
    a.gx = static_cast<int>((a.M + 16 * RT - 1) / (16 * RT));
    a.gy = (a.n + 16 * CT - 1) / (16 * CT);
    const int64_t grid = static_cast<int64_t>(a.gx) * a.gy;
    hipLaunchKernelGGL((mmq_kernel<F, RT, CT, NW, G>), dim3(static_cast<unsigned>(grid)), dim3(NW * kWave), 0, st,
                       a);
    return check_launch();
  }
}

template <class F, int NW, int G>
int launch_waves(const MmqArgs& a, int rt, int ct, hipStream_t st) {
  switch (rt * 10 + ct) {
    case 22: return launch_tile<F, 2, 2, NW, G>(a, st);
    case 21: return launch_tile<F, 2, 1, NW, G>(a, st);
    case 11: return launch_tile<F, 1, 1, NW, G>(a, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

template <class F, int G>
constexpr bool fits(int rt, int ct, int nw) {
  return rt == 2 ? (ct == 2 ? (nw == 8 ? tile_ok<F, 2, 2, 8, G>() : tile_ok<F, 2, 2, 4, G>())
                            : (nw == 8 ? tile_ok<F, 2, 1, 8, G>() : tile_ok<F, 2, 1, 4, G>()))
                 : (nw == 8 ? tile_ok<F, 1, 1, 8, G>() : tile_ok<F, 1, 1, 4, G>());
}

// Tile (row tiles x column tiles of 16 per workgroup): the largest tile that
// still gives every compute unit a workgroup (larger tiles re-read fewer
// weights and activations), has no more column tiles than n needs and fits
// the LDS and registers, else one tile. When the grid is no larger than the
// chip, eight waves split K instead of four, so each compute unit has more
// loads in flight (sixteen, at 128 registers per wave, measured slower:
// 4096x14336 Q4_K at 16 columns 16.3 -> 17.7 us).
template <class F, int G>
int launch_format(const MmqArgs& a, hipStream_t st) {
  static const int kTiles[][2] = {{2, 2}, {2, 1}, {1, 1}};
  const int64_t cus = device_cus();
  const int ct_max = (a.n + 15) / 16;
  int rt = 1, ct = 1;
  for (const auto& t : kTiles) {
    if (t[1] <= ct_max && groups(a, t[0], t[1]) >= cus && fits<F, G>(t[0], t[1], 4)) {
      rt = t[0];
      ct = t[1];
      break;
    }
  }
  int nw = groups(a, rt, ct) <= cus && fits<F, G>(rt, ct, 8) ? 8 : 4;
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_MMQ_TILE")) {
    rt = e[0] - '0';
    ct = e[2] - '0';
  }
  if (const char* e = getenv("MMVQ_MMQ_WAVES")) nw = atoi(e);
#endif
  switch (nw) {
    case 4: return launch_waves<F, 4, G>(a, rt, ct, st);
    case 8: return launch_waves<F, 8, G>(a, rt, ct, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

template <class F>
int launch_gated(const MmqArgs& a, hipStream_t st) {
  return a.Wg ? launch_format<F, 2>(a, st) : launch_format<F, 1>(a, st);
}

}  // namespace

int launch_mmq(int type, const MmqArgs& a, hipStream_t st) {
  switch (type) {
    case 12: return launch_gated<Q4K>(a, st);
    case 14: return launch_gated<Q6K>(a, st);
    case 2: return launch_gated<Q40>(a, st);
    case 8: return launch_gated<Q80>(a, st);
    case 3: return launch_gated<Q41>(a, st);
    case 6: return launch_gated<Q50>(a, st);
    case 7: return launch_gated<Q51>(a, st);
    case 13: return launch_gated<Q5K>(a, st);
    default: return MMVQ_ERR_TYPE;
  }
}

}  // namespace qmv
