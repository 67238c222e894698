// plan.hpp - launch shape and per-lane row window of the MMVQ kernels.
//
// Pure integer arithmetic shared by the host launcher, the kernels and the
// host model of the kernels' addressing (which checks every load of every
// lane against the buffers on the CPU).
#pragma once

#include "common.hpp"

namespace qmv {

// Waves per compute unit the row split aims for: enough to keep every
// CU's share of the matrix in flight in one round of resident waves.
#ifndef QMV_TARGET_WAVES_PER_CU
#define QMV_TARGET_WAVES_PER_CU 6
#endif

struct Shape {
  int units;            // units per row
  int chunks;           // K-chunks a team walks per row (1: a lane per unit)
  int slots;            // rows a team covers per step (P)
  int team_lanes;       // lanes per team (whole waves)
  int teams_per_block;
  int rows;             // rows per slot and pass (R)
  int passes;           // passes per team: the team owns passes * R * P rows
  int depth;            // pipelined rows (0: all rows' loads issued first)
  int64_t teams, blocks;
};

inline int pow2floor(int64_t v) {
  int p = 1;
  while (static_cast<int64_t>(p) * 2 <= v) p *= 2;
  return p;
}

// Longest row the kernels take, in units (32-bit lane offsets within a row
// and activation column stay far from overflow: Q6_K rows of 2^24 units
// are 880 MB).
constexpr int64_t kMaxUnitsPerRow = int64_t(1) << 24;

// Rows per team of a chunked launch (rows longer than a team: every row
// loops over its chunks, reloading the activation slice of each).
constexpr int kChunkRows = 4;

// Unit of lane lt in chunk c of a chunked team of TL lanes; lanes past the
// row's end re-read its last unit and are inactive.
__host__ __device__ __forceinline__ int chunk_unit(int lt, int c, int TL, int units, bool& active) {
  const int u = c * TL + lt;
  active = u < units;
  return active ? u : units - 1;
}

// Team layout and rows per team for an M-row matrix whose rows hold `units`
// units:
//  * chunks: rows of more than kLaunchBound units are walked in the fewest
//    chunks of at most kLaunchBound lanes, the team as wide as one chunk
//    (whole waves), at most kChunkRows rows per team and one pass;
//  * slots P = 2 when a row's units fill whole waves only in pairs (e.g.
//    224 units), else 1 (idle lanes pad the last wave);
//  * rows per slot and team: a power of two with rows * P <= M, sized for
//    about `target_waves` waves per CU (force_rows > 0 overrides the size,
//    for tuning), at most rmax * max_passes;
//  * rows per pass R: at most rmax (register budget); a team that owns more
//    rows takes them in passes of R (so the grid stays one round of resident
//    waves when the registers cap the rows of a pass).
inline Shape plan_rows(int64_t M, int units, int rmax, int64_t cus, int target_waves, int64_t force_rows,
                       int max_passes = 1) {
  Shape s;
  s.units = units;
  s.chunks = units > kLaunchBound ? (units + kLaunchBound - 1) / kLaunchBound : 1;
  const int lanes = (units + s.chunks - 1) / s.chunks;     // units per chunk
  s.slots = (s.chunks == 1 && units % kWave != 0 && (2 * units) % kWave == 0 && 2 * units <= kLaunchBound &&
             M >= 2) ? 2 : 1;
  s.team_lanes = (s.slots * lanes + kWave - 1) / kWave * kWave;
  const int tw = s.team_lanes / kWave;
  s.teams_per_block = s.team_lanes >= 256 ? 1 : 256 / s.team_lanes;
  int64_t want = force_rows > 0 ? force_rows : M * tw / (cus * target_waves * s.slots);
  int r = pow2floor(want < 1 ? 1 : want);
  if (s.chunks > 1) max_passes = 1;
  if (s.chunks > 1 && rmax > kChunkRows) rmax = kChunkRows;
  if (r > rmax * max_passes) r = rmax * max_passes;
  if (static_cast<int64_t>(r) * s.slots > M) r = pow2floor(M / s.slots);
  s.passes = r > rmax ? r / rmax : 1;
  s.rows = r / s.passes;
  const int64_t rp = static_cast<int64_t>(r) * s.slots;
  s.teams = (M + rp - 1) / rp;
  s.blocks = (s.teams + s.teams_per_block - 1) / s.teams_per_block;
  s.depth = 0;
  return s;
}

// Pipeline depth of a single-pass launch with R >= 8 rows per slot, for the
// fp32-activation forms of the lane layouts where it was measured to pay:
// few waves per CU, each owning many rows (4096x14336 Q4_K, 7 waves per CU:
// depth 4 -> 8.74 us against 9.90 with all 16 rows issued first; 4096x4096,
// 2 waves per CU: depth 8). With many waves per CU (the Q6_K LM head: 62)
// the hardware already overlaps the waves' loads and arithmetic and the
// shallower queue only costs (84.5 -> 95.5 us), as it did for Q8_0
// 4096x14336 (14.7 -> 16.2 us). max_per_cu: the most waves per CU at which
// the layout pipelines (layout_depth_cap; 0: never). Instantiated depths: 4
// and 8.
inline int plan_depth(const Shape& s, int64_t cus, int max_per_cu) {
  if (max_per_cu <= 0 || s.passes != 1 || s.rows < 8) return 0;
  const int64_t waves = s.teams * (s.team_lanes / kWave);
  const int64_t per_cu = (waves + cus - 1) / cus;
  if (per_cu > max_per_cu) return 0;
  const int d = per_cu >= 5 ? 4 : 8;
  return d < s.rows ? d : 0;
}

// Teams of fewer than 256 lanes share a workgroup; when that would leave
// compute units without one (4096x4096 Q4_K at 16 rows per team: 256
// two-wave teams in 128 workgroups), every team takes a workgroup of its own.
inline Shape spread_teams(Shape s, int64_t cus) {
  if (s.teams_per_block > 1 && s.blocks < cus) {
    s.teams_per_block = 1;
    s.blocks = s.teams;
  }
  return s;
}

// Shape of a rows-kernel launch: plan_rows; for the fp32-activation forms of
// a pipelined layout (depth_cap = layout_depth_cap > 0), at one column the
// most rows per team that still leaves a team per CU (each team quantizes
// the whole activation; 4096x4096 Q4_K: 4 rows per team 5.42 us, 16 rows at
// depth 8: 4.82), and the pipelined rows of plan_depth for every
// single-pass launch.
// rmax_flat (0: rmax): the most rows a team issues all at once, when rmax
// counts on pipelined rows (only DEPTH + 1 rows' weights live): a launch
// left without pipelining is planned again within it.
inline Shape plan_launch(int64_t M, int units, int rmax, int64_t cus, int max_passes, bool xf, int nc,
                         int64_t force_rows, int depth_cap, int rmax_flat = 0) {
  Shape s = plan_rows(M, units, rmax, cus, QMV_TARGET_WAVES_PER_CU, force_rows, max_passes);
  if (xf && depth_cap > 0) {
    if (nc == 1 && s.passes == 1 && force_rows == 0) {
      const int64_t per_cu = M / (cus * s.slots);
      const Shape t = plan_rows(M, units, rmax, cus, QMV_TARGET_WAVES_PER_CU, per_cu > 0 ? per_cu : 1, 1);
      if (t.rows > s.rows) s = t;
    }
    s.depth = plan_depth(s, cus, depth_cap);
  }
  if (s.depth == 0 && rmax_flat > 0 && s.rows > rmax_flat)
    s = plan_rows(M, units, rmax_flat, cus, QMV_TARGET_WAVES_PER_CU, force_rows, max_passes);
  return spread_teams(s, cus);
}

// Lane layouts whose fp32-activation launches take pipelined rows, where
// measured faster, and up to how many waves per CU: the half-chunk Q4_K
// layout (8, above), Q4_1, Q5_1 and Q5_K (16; at 4096x14336, one column:
// Q4_1 9.82 -> 9.62 us at 7 waves per CU, Q5_1 12.08 -> 10.68 at 7, Q5_K
// 13.82 -> 11.92 at 14). The others keep every row issued first (Q5_0
// measured slower pipelined: 13.4 -> 16.0 us; Q8_0 and Q6_K see plan_depth).
template <class F>
constexpr int layout_depth_cap() {
  if (F::kType == 12 && F::kUnitsPerBlock == 8) return 8;
  return (F::kType == 3 || F::kType == 7 || F::kType == 13) ? 16 : 0;
}
template <class F>
constexpr bool layout_pipelined() { return layout_depth_cap<F>() > 0; }

// Largest rows per slot (register budget) of an instantiation.
template <class F>
constexpr int rows_per_pass(int nc, int g) {
  int r = 1;
  if (F::kType == 14) r = nc == 1 ? 8 : (nc == 2 ? 4 : (nc <= 4 ? 2 : 1));   // Q6_K: 19 + 24n words
  else if (F::kType == 12 && F::kUnitsPerBlock == 4)
    r = nc == 1 ? 8 : (nc <= 4 ? 4 : 2);                                      // Q4_K whole chunks: 12 + 20n words
  else if (F::kType == 12) r = nc == 1 ? 16 : (nc <= 4 ? 8 : 4);              // Q4_K: 8 + 12n words
  else if (F::kType == 13) r = nc == 1 ? 8 : (nc <= 4 ? 4 : 2);               // Q5_K: 12 + 12n words
  else r = nc == 1 ? 16 : (nc <= 4 ? 8 : 4);                                 // Q4_0: 5 + 10n words
  return g == 2 ? (r > 1 ? r / 2 : 1) : r;
}

// Most rows per slot a mat-vec launch uses: the register budget, except the
// plain half-chunk Q4_K, Q8_0, Q4_1, Q5_0, Q5_1 and Q5_K mat-vecs at one
// q8_1 column, where teams of at most 4 rows measured faster (more, shorter
// teams: Q4_K 4096x14336 8.65 -> 8.05 us, 14336x4096 8.58 -> 7.75 us; Q8_0
// 4096x14336 13.25 -> 12.83 us; at 4096x14336 Q4_1 8.40 -> 8.13, Q5_0
// 10.19 -> 9.27, Q5_1 10.38 -> 9.68, Q5_K 10.60 -> 9.70 us); their fused
// fp32 forms keep larger teams, which re-read the fp32 activation fewer
// times. The result does not depend on the rows per team: every output's
// team sum runs the same reduction tree.
template <class F>
constexpr bool launch_short_teams(bool xf, int nc, int g) {
  const bool short_teams = (F::kType == 12 && F::kUnitsPerBlock == 8) || F::kType == 8 || F::kType == 3 ||
                           F::kType == 6 || F::kType == 7 || F::kType == 13;
  return short_teams && !xf && nc == 1 && g == 1 && rows_per_pass<F>(nc, g) > 4;
}

// ... and the single-column fp32 Q5_K form, whose 16-row teams (pipelined:
// only DEPTH + 1 rows' weights live; 4096x14336 11.4-11.8 -> 10.5-10.6 us
// against 8-row teams) re-quantize the activation half as often.
template <class F>
constexpr int launch_max_rows(bool xf, int nc, int g) {
  if (launch_short_teams<F>(xf, nc, g)) return 4;
  if (F::kType == 13 && xf && nc == 1 && g == 1) return 16;
  return rows_per_pass<F>(nc, g);
}

// Passes per team a mat-vec launch may use (rows kernels take a pass count of
// 1, 2 or 4): where the register budget caps the rows of a pass below
// what the row split wants, the team can take its rows in double-buffered
// passes instead of the grid growing into more teams. Fewer, longer teams
// pay off where each team has a large fixed cost: the fp32-activation
// forms, where every team reads and quantizes the whole activation
// (Q4_K 4096x14336 n = 2 / 4 / 8: 15.3 / 22.4 / 59 -> 12.0 / 17.0 / 38.6 us),
// and Q6_K, whose one-wave teams at K = 4096 make a grid of many rounds
// (128256x4096 n = 2: 94.6 -> 85.6 us). The q8_1 forms of the other formats
// and the gate/up forms measured slower with passes (Q4_K n = 2: 9.6 ->
// 10.6 us), and the Q6_K gate/up forms spill with them. Two passes hold two
// passes' weights in registers, which fits without spilling from two
// columns on (Q6_K: two to six).
constexpr int kMaxRowPasses = 4;

template <class F>
constexpr int launch_max_passes(bool xf, int nc, int g) {
  const bool fits = nc >= 2 && !(F::kType == 14 && nc >= 7);
  const bool pays = g == 1 && (F::kType == 14 || xf);
  return fits && pays ? kMaxRowPasses : 1;
}

// Rows per slot an expert block owns (taken in passes when its token count
// leaves registers for fewer): the register budget at one token, except the
// whole-chunk Q4_K kernels: with q8_1 activations the gate/up kernel's 8-row
// blocks measured faster than 4 (8-expert gate/up MoE: ~100 -> ~92 us; 2
// rows: ~138, 16: ~100); with fp32 activations, where every block
// re-quantizes its tokens, 32-row blocks (gate/up: 131 -> 112 us, 16 rows:
// 126, 64: 127; up only: 95 -> 67 us).
template <class F>
constexpr int id_block_rows(int g, bool xf = false) {
  if (F::kType == 12 && F::kUnitsPerBlock == 4) return xf ? 32 : (g == 2 ? 8 : rows_per_pass<F>(1, g));
  return rows_per_pass<F>(1, g);
}

// Rows per pass of an expert block with nc tokens: the register budget for
// nc columns, at most RB. When the block takes its rows in (double-buffered)
// passes and holds its fp32 activation slice raw across the weight loads,
// the two passes' weights plus the raw slice are kept within 160 registers
// (Q4_K whole chunks, one token: 8 rows -> 4, gate/up 4 -> 2; they spilled).
template <class F>
constexpr int id_rows_n(int nc, int RB, int G, bool XF) {
  int r = rows_per_pass<F>(nc, G) < RB ? rows_per_pass<F>(nc, G) : RB;
  constexpr int wt_words = static_cast<int>(sizeof(typename F::Wt) / 4);
  if (XF && nc * F::kXWords <= 64 && r < RB)
    while (r > 1 && 2 * r * G * wt_words + nc * F::kXWords > 160) r /= 2;
  return r;
}

// Row window of one team and the unit / slot of one of its lanes.
// The team owns rows [first, first + RP); the last team's window is moved
// back to end at row M-1 (M >= RP), and rows of the window below `first`
// (owned by the previous team) are skipped at the store. Lanes past the
// units of their slot are idle: they re-read the last unit and contribute 0.
struct Window {
  int64_t row0;     // first row of the window
  int64_t skip;     // leading window rows not stored by this team
  int slot;         // row slot of the lane (0 .. P-1)
  int unit;         // unit the lane loads (valid even when idle)
  bool active;
};

__host__ __device__ __forceinline__ Window team_window(int64_t team, int lt, int R, int P, int units,
                                                       int64_t M) {
  Window w;
  const int64_t rp = static_cast<int64_t>(R) * P;
  const int64_t first = team * rp;
  w.row0 = first + rp <= M ? first : M - rp;
  w.skip = first - w.row0;
  w.slot = (P == 1 || lt < units) ? 0 : 1;       // P <= 2
  const int lu = lt - w.slot * units;
  w.active = lu < units;
  w.unit = w.active ? lu : units - 1;
  return w;
}

}  // namespace qmv
