// mmq_launch.hpp - launch of the many-column (MFMA) kernel: tile and wave
// choice, instantiated by kernels_mmq.hip (q8_1 columns) and
// kernels_mmq_f32.hip (fp32 columns, quantized in the kernel).
#pragma once

#include <cstdlib>

#include "launch.hpp"
#include "mmq_kernel.hpp"

namespace qmv {

inline int64_t mmq_groups(const MmqArgs& a, int rt, int ct) {
  return ((a.M + 16 * rt - 1) / (16 * rt)) * ((a.n + 16 * ct - 1) / (16 * ct));
}

// Tiles of the gate/up form: every tile whose two accumulator sets and
// staging buffers fit the registers without spilling.
template <class F, int RT, int CT>
constexpr bool mmq_glu_tile() { return true; }

// The fused form (XF) stages 16 columns per workgroup: its staging
// registers grow with the columns (32 fp32 values per lane and block).
template <class F, int RT, int CT, int NW, int G, bool XF>
constexpr bool tile_ok() {
  return mmq_fits<F, RT, CT, NW, G>() && (G == 1 || mmq_glu_tile<F, RT, CT>()) && (!XF || CT == 1);
}

template <class F, int RT, int CT, int NW, int G, bool XF>
int launch_tile(MmqArgs a, hipStream_t st) {
  if constexpr (!tile_ok<F, RT, CT, NW, G, XF>()) {
    return MMVQ_ERR_SHAPE;
  } else {
    a.gx = static_cast<int>((a.M + 16 * RT - 1) / (16 * RT));
    a.gy = (a.n + 16 * CT - 1) / (16 * CT);
    const int64_t grid = static_cast<int64_t>(a.gx) * a.gy;
    hipLaunchKernelGGL((mmq_kernel<F, RT, CT, NW, G, XF>), dim3(static_cast<unsigned>(grid)), dim3(NW * kWave), 0, st,
                       a);
    return check_launch();
  }
}

template <class F, int NW, int G, bool XF>
int launch_waves(const MmqArgs& a, int rt, int ct, hipStream_t st) {
  switch (rt * 10 + ct) {
    case 22: return launch_tile<F, 2, 2, NW, G, XF>(a, st);
    case 21: return launch_tile<F, 2, 1, NW, G, XF>(a, st);
    case 11: return launch_tile<F, 1, 1, NW, G, XF>(a, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

template <class F, int G, bool XF>
constexpr bool mmq_tile_fits(int rt, int ct, int nw) {
  return rt == 2 ? (ct == 2 ? (nw == 8 ? tile_ok<F, 2, 2, 8, G, XF>() : tile_ok<F, 2, 2, 4, G, XF>())
                            : (nw == 8 ? tile_ok<F, 2, 1, 8, G, XF>() : tile_ok<F, 2, 1, 4, G, XF>()))
                 : (nw == 8 ? tile_ok<F, 1, 1, 8, G, XF>() : tile_ok<F, 1, 1, 4, G, XF>());
}

// Tile (row tiles x column tiles of 16 per workgroup): the largest tile that
// still gives every compute unit a workgroup (larger tiles re-read fewer
// weights and activations), has no more column tiles than n needs and fits
// the LDS and registers, else one tile. When the grid is no larger than the
// chip, eight waves split K instead of four, so each compute unit has more
// loads in flight (sixteen, at 128 registers per wave, measured slower:
// 4096x14336 Q4_K at 16 columns 16.3 -> 17.7 us). The fp32 form (XF) takes
// the q8_1 form's row tiles and wave count with one column tile: each
// output then sums the same partial products in the same order, so the two
// forms agree bit for bit.
template <class F, int G>
constexpr bool mmq_f32_tiles_cover() {
  return (!tile_ok<F, 2, 1, 4, G, false>() || tile_ok<F, 2, 1, 4, G, true>()) &&
         (!tile_ok<F, 2, 1, 8, G, false>() || tile_ok<F, 2, 1, 8, G, true>()) &&
         (!tile_ok<F, 1, 1, 4, G, false>() || tile_ok<F, 1, 1, 4, G, true>()) &&
         (!tile_ok<F, 1, 1, 8, G, false>() || tile_ok<F, 1, 1, 8, G, true>()) &&
         (!tile_ok<F, 2, 2, 4, G, false>() || tile_ok<F, 2, 1, 4, G, true>()) &&
         (!tile_ok<F, 2, 2, 8, G, false>() || tile_ok<F, 2, 1, 8, G, true>());
}

template <class F, int G, bool XF>
int launch_format(const MmqArgs& a, hipStream_t st) {
  static_assert(!XF || mmq_f32_tiles_cover<F, G>(), "fp32 form lacks a tile of the q8_1 form");
  static const int kTiles[][2] = {{2, 2}, {2, 1}, {1, 1}};
  const int64_t cus = device_cus();
  const int ct_max = (a.n + 15) / 16;
  int rt = 1, ct = 1;
  for (const auto& t : kTiles) {
    if (t[1] <= ct_max && mmq_groups(a, t[0], t[1]) >= cus && mmq_tile_fits<F, G, false>(t[0], t[1], 4)) {
      rt = t[0];
      ct = t[1];
      break;
    }
  }
  int nw = mmq_groups(a, rt, ct) <= cus && mmq_tile_fits<F, G, false>(rt, ct, 8) ? 8 : 4;
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_MMQ_TILE")) {
    rt = e[0] - '0';
    ct = e[2] - '0';
  }
  if (const char* e = getenv("MMVQ_MMQ_WAVES")) nw = atoi(e);
#endif
  if (XF) ct = 1;
  switch (nw) {
    case 4: return launch_waves<F, 4, G, XF>(a, rt, ct, st);
    case 8: return launch_waves<F, 8, G, XF>(a, rt, ct, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

template <class F, bool XF>
int launch_gated(const MmqArgs& a, hipStream_t st) {
  return a.Wg ? launch_format<F, 2, XF>(a, st) : launch_format<F, 1, XF>(a, st);
}

template <bool XF>
int launch_mmq_form(int type, const MmqArgs& a, hipStream_t st) {
  switch (type) {
    case 12: return launch_gated<Q4K, XF>(a, st);
    case 14: return launch_gated<Q6K, XF>(a, st);
    case 2: return launch_gated<Q40, XF>(a, st);
    case 8: return launch_gated<Q80, XF>(a, st);
    case 3: return launch_gated<Q41, XF>(a, st);
    case 6: return launch_gated<Q50, XF>(a, st);
    case 7: return launch_gated<Q51, XF>(a, st);
    case 13: return launch_gated<Q5K, XF>(a, st);
    default: return MMVQ_ERR_TYPE;
  }
}

}  // namespace qmv
