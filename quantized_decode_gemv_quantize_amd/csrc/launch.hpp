// launch.hpp - host-side launch shapes for the MMVQ kernels.
//
// Shapes are derived from the problem, not from per-architecture tables:
//   * team lanes TL = units per row rounded up to whole waves (<= 512);
//   * rows per team: enough teams for about QMV_TARGET_WAVES_PER_CU resident waves per compute
//     unit, capped by the register budget R of the instantiation;
//   * teams per workgroup: enough for at least 256 threads when TL < 256.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>

#include "../../include/mmvq.h"
#include "mmvq_kernel.hpp"
#include "plan.hpp"

namespace qmv {

// Compute units of the current device (cached per device id).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <class F>
inline int units_per_row(int64_t K) {
  return static_cast<int>(K / F::kQK) * F::kUnitsPerBlock;
}

template <class F>
inline Shape make_shape(int64_t M, int64_t K, int rmax, int max_passes = 1) {
  int64_t force = 0;
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_FORCE_ROWS")) force = atoi(e);
  if (const char* e = getenv("MMVQ_MAX_PASSES")) max_passes = max_passes > 1 ? atoi(e) : 1;
#endif
  return plan_rows(M, units_per_row<F>(K), rmax, device_cus(), QMV_TARGET_WAVES_PER_CU, force, max_passes);
}

inline int check_launch() {
  return hipGetLastError() == hipSuccess ? MMVQ_OK : MMVQ_ERR_LAUNCH;
}

template <class F, bool XF, int NC, int G, int R, int P, int PASSES, int DEPTH = 0, bool KLOOP = false>
inline int launch_rows_r(const RowArgs& a, const Shape& s, hipStream_t st) {
  hipLaunchKernelGGL((mmvq_rows_kernel<F, NC, R, P, G, XF, PASSES, DEPTH, KLOOP>),
                     dim3(static_cast<unsigned>(s.blocks)), dim3(s.teams_per_block * s.team_lanes), 0, st, a);
  return check_launch();
}

// Rows longer than a team: one slot, one pass, at most kChunkRows rows.
template <class F, bool XF, int NC, int G>
inline int launch_rows_chunked(const RowArgs& a, const Shape& s, hipStream_t st) {
  constexpr int RMAX = rows_per_pass<F>(NC, G);
  if (s.slots != 1 || s.passes != 1 || s.depth != 0 || s.teams_per_block != 1) return MMVQ_ERR_SHAPE;
  switch (s.rows) {
    case 1: return launch_rows_r<F, XF, NC, G, 1, 1, 1, 0, true>(a, s, st);
    case 2: if constexpr (RMAX >= 2) return launch_rows_r<F, XF, NC, G, 2, 1, 1, 0, true>(a, s, st); break;
    case 4: if constexpr (RMAX >= 4) return launch_rows_r<F, XF, NC, G, 4, 1, 1, 0, true>(a, s, st); break;
    default: break;
  }
  return MMVQ_ERR_SHAPE;
}

// one team per workgroup, or teams of one or two waves several per
// workgroup; other team widths: not launched here (MMVQ_ERR_SHAPE)
template <class F, int R, int DEPTH, bool XF>
inline int launch_rows1(const RowArgs& a, const Shape& s, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(s.blocks)), block(static_cast<unsigned>(s.teams_per_block * s.team_lanes));
  if (s.teams_per_block == 1) hipLaunchKernelGGL((mmvq_rows1_kernel<F, R, DEPTH, XF, 0>), grid, block, 0, st, a);
  else if (s.team_lanes == kWave) hipLaunchKernelGGL((mmvq_rows1_kernel<F, R, DEPTH, XF, 1>), grid, block, 0, st, a);
  else if (s.team_lanes == 2 * kWave) hipLaunchKernelGGL((mmvq_rows1_kernel<F, R, DEPTH, XF, 2>), grid, block, 0, st, a);
  else return MMVQ_ERR_SHAPE;
  return check_launch();
}

inline bool rows1_team_ok(const Shape& s) {
  return s.teams_per_block == 1 || s.team_lanes == kWave || s.team_lanes == 2 * kWave;
}

// Single-pass launch, with the pipelined rows of plan_depth for the fp32
// forms (the q8_1 forms keep their short teams and issue every row first);
// one column, no gate and one slot, in teams of one workgroup or of one or
// two waves, take the lean kernel of that case.
template <class F, bool XF, int NC, int G, int R, int P>
inline int launch_rows_d(const RowArgs& a, const Shape& s, hipStream_t st) {
  if constexpr (NC == 1 && G == 1 && P == 1) {
    if (rows1_team_ok(s)) {
      if constexpr (XF && R >= 8 && layout_pipelined<F>()) {
        if (s.depth == 4) return launch_rows1<F, R, 4, true>(a, s, st);
        if constexpr (R > 8)
          if (s.depth == 8) return launch_rows1<F, R, 8, true>(a, s, st);
      }
      // (not Q6_K: its one-wave LM-head teams measured slower there, 73.5 ->
      // 75.2 us at 128256x4096 with q8_1 activations, 82.9 -> 84.8 with fp32)
      if constexpr (R >= 2 && F::kType != 14)
        if (s.depth == 0) return launch_rows1<F, R, 0, XF>(a, s, st);
    }
  }
  if constexpr (XF && R >= 8 && layout_pipelined<F>()) {
    if (s.depth == 4) return launch_rows_r<F, XF, NC, G, R, P, 1, 4>(a, s, st);
    if constexpr (R > 8)
      if (s.depth == 8) return launch_rows_r<F, XF, NC, G, R, P, 1, 8>(a, s, st);
  }
  if (s.depth != 0) return MMVQ_ERR_SHAPE;
  return launch_rows_r<F, XF, NC, G, R, P, 1>(a, s, st);
}

// Passes > 1 come only with R = the register budget (plan_rows).
template <class F, bool XF, int NC, int G, int R>
inline int launch_rows_p(const RowArgs& a, const Shape& s, hipStream_t st) {
  if constexpr (R == rows_per_pass<F>(NC, G) && launch_max_passes<F>(XF, NC, G) > 1) {
    static_assert(launch_max_passes<F>(XF, NC, G) == 4, "rows kernels instantiated for 2 and 4 passes");
    if (s.passes == 2)
      return s.slots == 2 ? launch_rows_r<F, XF, NC, G, R, 2, 2>(a, s, st) : launch_rows_r<F, XF, NC, G, R, 1, 2>(a, s, st);
    if (s.passes == 4)
      return s.slots == 2 ? launch_rows_r<F, XF, NC, G, R, 2, 4>(a, s, st) : launch_rows_r<F, XF, NC, G, R, 1, 4>(a, s, st);
  }
  if (s.passes != 1) return MMVQ_ERR_SHAPE;
  return s.slots == 2 ? launch_rows_d<F, XF, NC, G, R, 2>(a, s, st) : launch_rows_d<F, XF, NC, G, R, 1>(a, s, st);
}

template <class F, bool XF, int NC, int G>
inline int launch_rows_nc(RowArgs a, int64_t K, hipStream_t st) {
  constexpr int RMAX = launch_max_rows<F>(XF, NC, G);
  int64_t force = 0;
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_FORCE_ROWS")) force = atoi(e);
#endif
  Shape s = plan_launch(a.M, units_per_row<F>(K), launch_max_rows<F>(XF, NC, G), device_cus(),
                        launch_max_passes<F>(XF, NC, G), XF, NC, force, layout_depth_cap<F>(),
                        rows_per_pass<F>(NC, G));
#ifdef QMV_TUNING
  if (const char* e = getenv("MMVQ_DEPTH")) s.depth = XF ? atoi(e) : 0;
#endif
  a.units = s.units;
  a.team_lanes = s.team_lanes;
  a.teams_per_block = s.teams_per_block;
  if (s.chunks > 1) return launch_rows_chunked<F, XF, NC, G>(a, s, st);
  switch (s.rows) {
    case 1: return launch_rows_p<F, XF, NC, G, 1>(a, s, st);
    case 2: if constexpr (RMAX >= 2) return launch_rows_p<F, XF, NC, G, 2>(a, s, st); break;
    case 4: if constexpr (RMAX >= 4) return launch_rows_p<F, XF, NC, G, 4>(a, s, st); break;
    case 8: if constexpr (RMAX >= 8) return launch_rows_p<F, XF, NC, G, 8>(a, s, st); break;
    case 16: if constexpr (RMAX >= 16) return launch_rows_p<F, XF, NC, G, 16>(a, s, st); break;
    default: break;
  }
  return MMVQ_ERR_SHAPE;
}

template <class F, bool XF, int G>
inline int launch_rows(const RowArgs& a, int64_t K, int64_t n, hipStream_t st) {
  switch (n) {
    case 1: return launch_rows_nc<F, XF, 1, G>(a, K, st);
    case 2: return launch_rows_nc<F, XF, 2, G>(a, K, st);
    case 3: return launch_rows_nc<F, XF, 3, G>(a, K, st);
    case 4: return launch_rows_nc<F, XF, 4, G>(a, K, st);
    case 5: return launch_rows_nc<F, XF, 5, G>(a, K, st);
    case 6: return launch_rows_nc<F, XF, 6, G>(a, K, st);
    case 7: return launch_rows_nc<F, XF, 7, G>(a, K, st);
    case 8: return launch_rows_nc<F, XF, 8, G>(a, K, st);
    default: return MMVQ_ERR_SHAPE;
  }
}

template <class F, bool XF, int G, int RB, int P, bool KLOOP = false>
inline int launch_id_r(const RowArgs& a, const Shape& s, int n_experts, hipStream_t st) {
  const unsigned slices = static_cast<unsigned>(n_experts) + (a.Ws_up ? 1u : 0u);   // + shared expert
  hipLaunchKernelGGL((mmvq_id_kernel<F, RB, P, G, XF, KLOOP>), dim3(static_cast<unsigned>(s.blocks), slices),
                     dim3(s.teams_per_block * s.team_lanes), 0, st, a);
  return check_launch();
}

// Expert blocks own RB = id_block_rows rows per slot;
// matrices with fewer rows fall back to one row per slot.
template <class F, bool XF, int G>
inline int launch_id(RowArgs a, int64_t K, int n_experts, hipStream_t st) {
  constexpr int RB = id_block_rows<F>(G, XF);
  Shape s = make_shape<F>(a.M, K, RB);
  a.units = s.units;
  a.team_lanes = s.team_lanes;
  a.teams_per_block = s.teams_per_block;
  // rows longer than a team: one row per team, walked in chunks
  const bool full = s.chunks == 1 && static_cast<int64_t>(RB) * s.slots <= a.M;
  const int rb = full ? RB : 1;
  s.rows = rb;
  s.teams = (a.M + static_cast<int64_t>(rb) * s.slots - 1) / (static_cast<int64_t>(rb) * s.slots);
  s.blocks = (s.teams + s.teams_per_block - 1) / s.teams_per_block;
  if (s.chunks > 1) {
    if (s.slots != 1 || s.teams_per_block != 1) return MMVQ_ERR_SHAPE;
    return launch_id_r<F, XF, G, 1, 1, true>(a, s, n_experts, st);
  }
  if (full)
    return s.slots == 2 ? launch_id_r<F, XF, G, RB, 2>(a, s, n_experts, st)
                        : launch_id_r<F, XF, G, RB, 1>(a, s, n_experts, st);
  return s.slots == 2 ? launch_id_r<F, XF, G, 1, 2>(a, s, n_experts, st)
                      : launch_id_r<F, XF, G, 1, 1>(a, s, n_experts, st);
}

template <class F>
inline int launch_block_dots(const uint8_t* W, const uint8_t* y, int32_t* dots, int64_t M, int64_t K,
                             int64_t n, hipStream_t st) {
  const int64_t nblocks = K / F::kQK;
  const int64_t total = n * M * nblocks;
  const int64_t row_bytes = nblocks * F::kBlockBytes;
  const int64_t ycol_bytes = K / 32 * kQ8Bytes;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(mmvq_block_dots_kernel<F>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     W, y, dots, M, nblocks, row_bytes, ycol_bytes, n);
  return check_launch();
}

// Per-format entry points: one translation unit per format and activation
// type (q8_1 columns, or fp32 columns quantized in the kernel prologue).
struct Dispatch {
  int (*rows)(const RowArgs&, int64_t K, int64_t n, hipStream_t);
  int (*rows_glu)(const RowArgs&, int64_t K, int64_t n, hipStream_t);
  int (*id)(const RowArgs&, int64_t K, int n_experts, hipStream_t);
  int (*id_glu)(const RowArgs&, int64_t K, int n_experts, hipStream_t);
  int (*block_dots)(const uint8_t*, const uint8_t*, int32_t*, int64_t, int64_t, int64_t, hipStream_t);
  int qk, block_bytes, units_per_block;
};

// ID = false leaves the expert-indexed launchers out (set by the caller).
template <class F, bool XF, bool ID = true>
Dispatch make_dispatch() {
  Dispatch d;
  d.rows = [](const RowArgs& a, int64_t K, int64_t n, hipStream_t s) { return launch_rows<F, XF, 1>(a, K, n, s); };
  d.rows_glu = [](const RowArgs& a, int64_t K, int64_t n, hipStream_t s) {
    return launch_rows<F, XF, 2>(a, K, n, s);
  };
  d.id = nullptr;
  d.id_glu = nullptr;
  if constexpr (ID) {
    d.id = [](const RowArgs& a, int64_t K, int e, hipStream_t s) { return launch_id<F, XF, 1>(a, K, e, s); };
    d.id_glu = [](const RowArgs& a, int64_t K, int e, hipStream_t s) { return launch_id<F, XF, 2>(a, K, e, s); };
  }
  d.block_dots = launch_block_dots<F>;
  d.qk = F::kQK;
  d.block_bytes = F::kBlockBytes;
  d.units_per_block = F::kUnitsPerBlock;
  return d;
}

// Q4_K has two lane layouts: half chunks (Q4K: 32 weights per lane) and
// whole chunks (Q4K2: 64). The fp32-activation forms must equal quantize +
// q8_1 form bit for bit, so both forms of a call take the same layout:
//  * mat-vec (rows kernels): half chunks, whole chunks only for rows longer
//    than a team of half-chunk lanes holds. Whole chunks make the q8_1 form
//    faster at one column (14336x4096: 8.6 -> 7.9 us) but the fused form
//    slower (9.5 -> 11.2 us: twice the teams or row slots, each quantizing
//    the whole activation), and the fused form is the faster step;
//  * expert kernels: whole chunks (8-expert gate/up, q8_1 activations:
//    122 -> 107 us; the fused form 162 -> 198 us, where the two-launch form
//    is the faster step either way: every expert block re-quantizes its
//    tokens).
// The row limit is the whole-chunk one.
constexpr int64_t kQ4KHalfMaxK = static_cast<int64_t>(kLaunchBound) / Q4K::kUnitsPerBlock * Q4K::kQK;

// Expert-indexed Q4_K launchers (whole chunks), each activation type in a
// translation unit of its own.
int launch_id_q4k(const RowArgs& a, int64_t K, int n_experts, hipStream_t st);
int launch_id_glu_q4k(const RowArgs& a, int64_t K, int n_experts, hipStream_t st);
int launch_id_q4k_f32(const RowArgs& a, int64_t K, int n_experts, hipStream_t st);
int launch_id_glu_q4k_f32(const RowArgs& a, int64_t K, int n_experts, hipStream_t st);

template <bool XF>
Dispatch make_dispatch_q4k() {
  Dispatch d = make_dispatch<Q4K, XF, false>();
  d.rows = [](const RowArgs& a, int64_t K, int64_t n, hipStream_t s) {
    return K > kQ4KHalfMaxK ? launch_rows<Q4K2, XF, 1>(a, K, n, s) : launch_rows<Q4K, XF, 1>(a, K, n, s);
  };
  d.rows_glu = [](const RowArgs& a, int64_t K, int64_t n, hipStream_t s) {
    return K > kQ4KHalfMaxK ? launch_rows<Q4K2, XF, 2>(a, K, n, s) : launch_rows<Q4K, XF, 2>(a, K, n, s);
  };
  d.id = XF ? launch_id_q4k_f32 : launch_id_q4k;
  d.id_glu = XF ? launch_id_glu_q4k_f32 : launch_id_glu_q4k;
  // the integer dots through the layout the mat-vec takes for this K
  d.block_dots = [](const uint8_t* W, const uint8_t* y, int32_t* dots, int64_t M, int64_t K, int64_t n,
                    hipStream_t s) {
    return K > kQ4KHalfMaxK ? launch_block_dots<Q4K2>(W, y, dots, M, K, n, s)
                            : launch_block_dots<Q4K>(W, y, dots, M, K, n, s);
  };
  d.units_per_block = Q4K2::kUnitsPerBlock;
  return d;
}

const Dispatch& dispatch_q4_0();
const Dispatch& dispatch_q8_0();
const Dispatch& dispatch_q4_k();
const Dispatch& dispatch_q6_k();
const Dispatch& dispatch_q4_1();
const Dispatch& dispatch_q5_0();
const Dispatch& dispatch_q5_1();
const Dispatch& dispatch_q5_k();
const Dispatch& dispatch_q4_0_f32();
const Dispatch& dispatch_q8_0_f32();
const Dispatch& dispatch_q4_k_f32();
const Dispatch& dispatch_q6_k_f32();
const Dispatch& dispatch_q4_1_f32();
const Dispatch& dispatch_q5_0_f32();
const Dispatch& dispatch_q5_1_f32();
const Dispatch& dispatch_q5_k_f32();

int launch_quantize_q8_1(const float* x, uint8_t* y, int64_t K, int64_t n, int64_t ldx, hipStream_t st);
int launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t st);

struct MmqArgs;
int launch_mmq(int type, const MmqArgs& a, hipStream_t st);
int launch_mmq_f32(int type, const MmqArgs& a, hipStream_t st);   // a.x: fp32 columns

}  // namespace qmv
