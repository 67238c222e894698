// mmvq_kernel.hpp - the quantized mat-vec kernels for gfx950.
//
// Citations: [MMVQ §X] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时
// 一条量化权重如何被 dp4a 逐块点积", section X.
//
// Decomposition (CDNA4-first, not the pages' warp-per-K-slice tiling):
//   * A team of TL lanes (a whole number of waves) owns a row: lane i of the
//     team always handles unit i of the row (see formats.hpp), so it loads
//     its slice of the activation once and keeps it in registers for every
//     row and column. Weight reuse is 1, so weights never touch LDS.
//   * A team owns up to R consecutive rows. It issues the weight loads of
//     all its rows before any arithmetic (branch-free: rows past the end are
//     clamped and their results dropped), so each wave has R x 32 bytes per
//     lane in flight and the whole matrix is requested early. Where the
//     registers cap R, a team may own 2 or 4 times R rows and take them in
//     double-buffered passes (loads of pass p+1 issued before pass p is
//     computed), loading its activation slice once.
//   * Per row the lane decodes its unit once and forms one fp32 partial per
//     activation column with v_dot4_i32_i8 integer dots; scales are applied
//     per block after the integer dot [MMVQ §一次 vec_dot 的解剖].
//   * The R x n partials of every lane are summed over the team with a
//     transposed reduction (common.hpp): each exchange halves the values a
//     lane carries, then waves combine through LDS and one lane per output
//     applies the epilogue and stores [MMVQ §归约与写出, §融合].
//   * G = 1 plain product; G = 2 fused gate/up: both weight streams are
//     read in the same pass and the GLU is applied in the epilogue.
//   * Expert-indexed mode: blockIdx.y is the expert; the block gathers the
//     tokens routed to it (at most 8) and reads that expert's rows once for
//     all of them [MMVQ §MoE]. A team owns RB rows and takes them in passes
//     of as many rows as the registers hold for the block's token count.
//   * XF = true takes fp32 activations and quantizes the lane's slice to
//     q8_1 in registers (formats.hpp load_x / quant_x), with the arithmetic
//     of the stand-alone quantizer: the same codes and scales, so the result
//     equals quantize-then-multiply bit for bit, without the q8_1 round trip
//     through memory or the second launch [MMVQ §激活的量化, §融合]. When
//     the raw values of all columns fit the register budget, the fp32 loads
//     go out first, then the weight loads, and the quantization runs while
//     the weights are in flight; otherwise each column is quantized before
//     the weight loads are issued.
#pragma once

#include "common.hpp"
#include "formats.hpp"
#include "plan.hpp"

namespace qmv {


struct RowArgs {
  const uint8_t* W;          // up / plain weights (expert 0 in id mode)
  const uint8_t* Wg;         // gate weights (G = 2)
  const uint8_t* y;          // q8_1 columns (XF = false)
  const float* x;            // fp32 columns (XF = true), column stride ldx
  float* out;
  const int32_t* ids;        // id mode: n_tokens x top_k
  int64_t M;
  int64_t row_bytes;
  int64_t ycol_bytes;
  int64_t ldx;               // elements between fp32 columns
  int64_t expert_stride;
  int units;                 // units per row
  int team_lanes;            // TL: multiple of 64
  int teams_per_block;       // the workgroup is teams_per_block * TL lanes
  int glu_op;                // GLU of the gate forms (see glu())
  int n_tokens;              // id mode
  int top_k;                 // id mode
  // epilogue [MMVQ §融合]: up = up*up_scale[e] + up_bias[e*M + r], the same
  // for the gate, then the GLU; NULL pointers are skipped (e = expert in id
  // mode, else 0)
  const float* up_bias;
  const float* gate_bias;
  const float* up_scale;
  const float* gate_scale;
  float glu_limit;
  // id mode: shared expert in the extra grid slice blockIdx.y == n_experts
  int n_experts;
  const uint8_t* Ws_up;
  const uint8_t* Ws_gate;
  float* shared_out;
};

// GLU ops of the fused epilogue [MMVQ §融合] (the page names them, its
// switch calls the device functions without their bodies): 0 gate*up,
// 1 silu(gate)*up, 2 gelu(gate)*up with gelu in its tanh form
// 0.5*z*(1 + tanh(sqrt(2/pi)*(z + 0.044715*z^3))), 3 the clamped SwiGLU
// published with the gpt-oss models, g'*sigmoid(1.702*g')*(u'+1) with
// g' = min(gate, 7), u' = clamp(up, -7, 7) (the page passes it no
// parameter), 4 silu(g')*u' with the caller's limit in the same clamps.
__device__ __forceinline__ float glu(int op, float gate, float up, float limit) {
  switch (op) {
    case 1: return gate / (1.0f + __expf(-gate)) * up;
    case 2: {
      const float t = tanhf(0.7978845608028654f * (gate + 0.044715f * gate * gate * gate));
      return 0.5f * gate * (1.0f + t) * up;
    }
    case 3: {
      const float g = fminf(gate, 7.0f), u = fminf(fmaxf(up, -7.0f), 7.0f);
      return g / (1.0f + __expf(-1.702f * g)) * (u + 1.0f);
    }
    case 4: {
      const float g = fminf(gate, limit), u = fminf(fmaxf(up, -limit), limit);
      return g / (1.0f + __expf(-g)) * u;
    }
    default: return gate * up;
  }
}

// Column descriptor: which q8_1 column feeds activation slot j, and where
// its results go (one output slot per column in plain mode; in id mode a
// token may feed several slots of the same expert, bitmask over k).
struct Cols {
  int n;                       // active columns
  int tok[kMaxCols];
  uint64_t slots[kMaxCols];    // id mode: bit k set -> out slot tok*top_k + k
};

// LDS for the cross-wave step: G planes x waves x (values per lane group).
template <int G, int V>
struct RedLds {
  float v[G][kMaxWavesPerBlock * V];
};

// P row slots: when the units of a row fill only part of the last wave,
// the team covers P rows at once (slot s = lane / units), so a 224-unit row
// pair fills 7 waves exactly. Lane values are indexed
// (column j, row i*P + slot); a lane holds zeros for the other slots, and
// the team reduction sums each value over the lanes of its own slot.
// PASSES: the team owns PASSES * R * P consecutive rows and takes them R * P
// at a time, loading its activation slice once (the expert-indexed kernel
// uses this to keep R*P rows of loads in flight whatever the column count).
// DEPTH (single pass only; 0 = off): software-pipelined rows. Only the first
// DEPTH rows' loads are issued up front; row i is computed as soon as it has
// landed and only then are row i + DEPTH's loads issued. Without it a wave
// issues all R rows' loads first, and under a saturated memory system those
// issues stall (the queue only takes a load when an older one drains), so
// the wave sits in its load issues while its first rows have landed and then
// computes all R rows after its last row arrives; with it the arithmetic
// runs while the later rows stream.
// KLOOP (one slot, one pass, no pipelining): rows with more units than a
// team has lanes. The team walks the row in chunks of TL units; in chunk c
// lane lt handles unit c*TL + lt with that unit's activation slice, and
// adds its chunks' partials in chunk order before the team reduction (the
// pages split K over the warps of a block the same way, [MMVQ §kernel 的形状]).
template <class F, int NC, int R, int P, int G, bool ID, bool XF, int VMAX, int PASSES = 1, int DEPTH = 0,
          bool KLOOP = false>
__device__ __forceinline__ void rows_body(const RowArgs& a, const Cols& cols,
                                          const uint8_t* Wbase, const uint8_t* Wgbase,
                                          RedLds<G, VMAX>& red) {
  constexpr int RP = R * P;                 // rows per pass
  constexpr int V = pow2ceil(NC * RP);
  static_assert(V <= VMAX, "LDS sized for fewer values");
  // Every scalar argument the weight loads and the epilogue need, read in
  // the kernel's first batch of argument loads: left to the compiler, some
  // were loaded after the activation loads (one more scalar round trip before
  // the weight stream) or at the store (one at the end of every wave).
  // (Input-only operands: the pointers keep their global address space.)
  const uint8_t* Wb = Wbase;
  const uint8_t* Wgb = Wgbase;
  const float *up_scale = a.up_scale, *up_bias = a.up_bias, *gate_scale = a.gate_scale, *gate_bias = a.gate_bias;
  asm volatile("" ::"s"(Wb), "s"(Wgb), "s"(up_scale), "s"(up_bias), "s"(gate_scale), "s"(gate_bias));
  const int tid = threadIdx.x;
  const int TL = a.team_lanes;
  // team index and row window are wave-uniform (teams are whole waves):
  // keep them scalar so row addresses are SGPR base + per-lane offset
  const int teams_per_block = a.teams_per_block;
  // one team per workgroup (every team of 256 lanes or more) needs no
  // division by the team size before the first loads can be issued
  const int team_local = teams_per_block == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / TL);
  const int lt = tid - team_local * TL;
  const int64_t team = static_cast<int64_t>(blockIdx.x) * teams_per_block + team_local;
  const Window win = team_window(team, lt, R * PASSES, P, a.units, a.M);
  int64_t row0 = win.row0, skip = win.skip;   // of the current pass
  const int slot = win.slot;
  bool active = win.active;        // the lane's unit and its constants
  int u = win.unit;                // (per chunk with KLOOP)
  const int lane = lane_id();
  typename F::Lane L = F::lane(u);
  const int64_t step = static_cast<int64_t>(P) * a.row_bytes;

  // ---- activation slice of every column (zero for idle lanes) -----------
  // Only the loads are issued here; what needs their data runs after the
  // weight loads have been issued, so no wave waits for its activation
  // before its weight stream is in flight. XE: fp32 values held in
  // registers across the weight loads (else quantized up front).
  constexpr bool XE = XF && NC * F::kXWords <= 64;
  typename F::Act act[NC];
  typename F::XRaw xr[XE ? NC : 1];
  auto load_act = [&]() QMV_INLINE {
    if constexpr (XF && !XE) {
      // compile-time column index: at 8 columns the body exceeds what the
      // loop unroller takes, and a runtime index would put act[] in scratch
      static_for<0, NC>([&](auto jc) QMV_INLINE {
        constexpr int j = decltype(jc)::value;
        typename F::XRaw t;
        F::load_x(t, a.x + cols.tok[j] * a.ldx, u);
        F::quant_x(act[j], t);
        if (!active) F::zero_act(act[j]);
      });
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if constexpr (XE) F::load_x(xr[j], a.x + cols.tok[j] * a.ldx, u);
        else F::issue_act(act[j], a.y + cols.tok[j] * a.ycol_bytes, u);
      }
    }
  };
  // the activation loads were issued before the weight loads, so they
  // retire first: this waits for them only
  auto finish_act = [&]() QMV_INLINE {
    if constexpr (XE) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        F::quant_x(act[j], xr[j]);
        if (!active) F::zero_act(act[j]);
      }
    } else if constexpr (!XF) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        F::finish_act(act[j]);
        if (!active) F::zero_act(act[j]);
      }
    }
  };

  // ---- issue all weight loads of a pass's rows ---------------------------
  // With several passes the weights are double-buffered: the loads of pass
  // p+1 are issued before pass p is computed, so a wave never waits for a
  // whole round trip between passes.
  constexpr int NB = PASSES > 1 ? 2 : 1;
  typename F::Wt wb[NB][R];
  typename F::Wt wgb[NB][G == 2 ? R : 1];
  // uniform row pointers; the slot's row is a per-lane 32-bit offset
  const uint32_t slot_off = static_cast<uint32_t>(slot * a.row_bytes);
  static_assert(DEPTH == 0 || (PASSES == 1 && DEPTH < R), "pipelined rows: one pass, depth below R");
  constexpr int FIRST = DEPTH > 0 ? DEPTH : R;      // rows issued up front
  auto issue = [&](typename F::Wt (&w)[R], typename F::Wt (&wg)[G == 2 ? R : 1], int64_t r0, int i0,
                   int i1) QMV_INLINE {
    const uint8_t* rp = Wb + r0 * a.row_bytes + i0 * step;
    const uint8_t* gp = (G == 2) ? Wgb + r0 * a.row_bytes + i0 * step : nullptr;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      F::load_wt(w[i], rp, slot_off, L);
      rp += step;
      if constexpr (G == 2) {
        F::load_wt(wg[i], gp, slot_off, L);
        gp += step;
      }
      // keep the loads in row order: row i's arithmetic then waits only for
      // rows 0..i (the vector memory counter retires loads in issue order)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- reduce over the team, epilogue, store -----------------------------
  using RM = ReduceMap<kWave, V>;
  auto store = [&](int idx, float up, float gate) QMV_INLINE {
    const int j = idx / RP, i = idx - j * RP;
    if (j >= NC || i < skip) return;
    const int64_t r = row0 + i;
    const int64_t e = ID ? static_cast<int64_t>(blockIdx.y) : 0;
    if (up_scale) up *= up_scale[e];
    if (up_bias) up += up_bias[e * a.M + r];
    if constexpr (G == 2) {
      if (gate_scale) gate *= gate_scale[e];
      if (gate_bias) gate += gate_bias[e * a.M + r];
    }
    const float v = (G == 2) ? glu(a.glu_op, gate, up, a.glu_limit) : up;
    if constexpr (ID) {
      // select column j's token and slots with compile-time indices
      uint64_t m = 0;
      int t = 0;
#pragma unroll
      for (int jj = 0; jj < NC; ++jj)
        if (jj == j) { m = cols.slots[jj]; t = cols.tok[jj]; }
      while (m) {
        const int k = __builtin_ctzll(m);
        m &= m - 1;
        a.out[(static_cast<int64_t>(t) * a.top_k + k) * a.M + r] = v;
      }
    } else {
      a.out[static_cast<int64_t>(j) * a.M + r] = v;
    }
  };
  // resync: a previous pass's readers must be done with the LDS first
  // (uniform: every team of the block runs the same passes)
  auto reduce_store = [&](float (&part)[G][V], bool resync) QMV_INLINE {
    team_reduce<kWave, G, V>(part, lane);
    if (TL == kWave) {
      if (RM::representative(lane)) {
#pragma unroll
        for (int pos = 0; pos < RM::kPerLane; ++pos) {
          const int idx = RM::index(lane, pos);
          store(idx, part[0][pos], G == 2 ? part[G - 1][pos] : 0.0f);
        }
      }
    } else {
      const int wave = tid / kWave;
      if (resync) __syncthreads();
      if (RM::representative(lane)) {
#pragma unroll
        for (int pos = 0; pos < RM::kPerLane; ++pos) {
          const int idx = RM::index(lane, pos);
#pragma unroll
          for (int p = 0; p < G; ++p) red.v[p][wave * V + idx] = part[p][pos];
        }
      }
      __syncthreads();
      const int tw = TL / kWave;
      const int wave0 = team_local * tw;
      for (int idx = lt; idx < NC * RP; idx += TL) {
        float s[G];
#pragma unroll
        for (int p = 0; p < G; ++p) {
          s[p] = 0.0f;
          for (int k = 0; k < tw; ++k) s[p] += red.v[p][(wave0 + k) * V + idx];
        }
        store(idx, s[0], s[G - 1]);
      }
    }
  };

  if constexpr (KLOOP) {
    static_assert(P == 1 && PASSES == 1 && DEPTH == 0, "chunked rows: one slot, one pass, no pipelining");
    const int chunks = (a.units + TL - 1) / TL;
    float part[G][V];
#pragma unroll
    for (int p = 0; p < G; ++p)
#pragma unroll
      for (int k = 0; k < V; ++k) part[p][k] = 0.0f;
    typename F::Wt (&w)[R] = wb[0];
    typename F::Wt (&wg)[G == 2 ? R : 1] = wgb[0];
    for (int c = 0; c < chunks; ++c) {
      u = chunk_unit(lt, c, TL, a.units, active);
      L = F::lane(u);
      load_act();
      __builtin_amdgcn_sched_barrier(0);
      issue(w, wg, row0, 0, R);
      finish_act();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        typename F::Dec dec;
        F::decode(w[i], dec, L);
#pragma unroll
        for (int j = 0; j < NC; ++j) part[0][j * R + i] += F::col_dot(dec, act[j]);
        if constexpr (G == 2) {
          F::decode(wg[i], dec, L);
#pragma unroll
          for (int j = 0; j < NC; ++j) part[1][j * R + i] += F::col_dot(dec, act[j]);
        }
      }
    }
    reduce_store(part, false);
    return;
  }

  load_act();
  __builtin_amdgcn_sched_barrier(0);
  issue(wb[0], wgb[0], row0, 0, FIRST);
  finish_act();

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
  if (pass > 0) {
    row0 += RP;
    skip -= RP;
  }
  if (pass + 1 < PASSES) issue(wb[(pass + 1) % NB], wgb[(pass + 1) % NB], row0 + RP, 0, R);
  typename F::Wt (&w)[R] = wb[pass % NB];
  typename F::Wt (&wg)[G == 2 ? R : 1] = wgb[pass % NB];
  // ---- per row: decode once, one partial per column ----------------------
  float part[G][V];
#pragma unroll
  for (int p = 0; p < G; ++p)
#pragma unroll
    for (int k = 0; k < V; ++k) part[p][k] = 0.0f;
  auto put = [&](int p, int j, int i, float v) QMV_INLINE {
    if constexpr (P == 1) {
      part[p][j * RP + i] = v;
    } else {
#pragma unroll
      for (int s = 0; s < P; ++s) part[p][j * RP + i * P + s] = slot == s ? v : 0.0f;
    }
  };
#pragma unroll
  for (int i = 0; i < R; ++i) {
    typename F::Dec dec;
    F::decode(w[i], dec, L);
#pragma unroll
    for (int j = 0; j < NC; ++j) put(0, j, i, F::col_dot(dec, act[j]));
    if constexpr (G == 2) {
      F::decode(wg[i], dec, L);
#pragma unroll
      for (int j = 0; j < NC; ++j) put(1, j, i, F::col_dot(dec, act[j]));
    }
    if constexpr (DEPTH > 0) {
      // row i's arithmetic stays ahead of the next issue
      __builtin_amdgcn_sched_barrier(0);
      if (i + DEPTH < R) issue(w, wg, row0, i + DEPTH, i + DEPTH + 1);
    }
  }

  reduce_store(part, PASSES > 1 && pass > 0);
  }   // passes
}

// The single-column mat-vec with one team of whole waves per workgroup and
// one row slot (a single decode token: the fused step with pipelined rows,
// XF, or the q8_1 form with every row issued first, DEPTH = 0): the same
// loads, arithmetic and reduction order as rows_body for that case (so the
// outputs equal rows_body's, and the fused form's quantize + the q8_1
// form's, bit for bit), with the general kernel's per-team bookkeeping left
// out: the team is the workgroup, the row window a clamp of blockIdx.x * R,
// the weight rows 32-bit offsets from the team's first row (one team's rows
// span less than 4 GB: at most 512 units of a row), the epilogue the up
// scale and bias. At 4096x14336 Q4_K the fused form measured 8.42-8.45 us
// against rows_body's 8.67-8.72 (experiment harness, same launch shape).
// TW = 0: one team per workgroup; TW > 0: teams of TW waves, as many per
// workgroup as it holds (the team index a compile-time division of the
// wave index).
template <class F, int R, int DEPTH, bool XF, int TW>
__global__ void __launch_bounds__(kLaunchBound) mmvq_rows1_kernel(RowArgs a) {
  static_assert(DEPTH >= 0 && DEPTH < R, "pipelined rows below R");
  constexpr int FIRST = DEPTH > 0 ? DEPTH : R;      // rows issued up front
  __shared__ float red[kMaxWavesPerBlock * R];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int team_local = TW > 0 ? wave / TW : 0;
  const int tw = TW > 0 ? TW : static_cast<int>(blockDim.x) / kWave;     // waves of the team
  const int lt = tid - team_local * TW * kWave;
  const int64_t team = TW > 0 ? static_cast<int64_t>(blockIdx.x) * (blockDim.x / (TW * kWave)) + team_local
                              : static_cast<int64_t>(blockIdx.x);
  const int units = a.units;
  const bool active = lt < units;
  const int u = active ? lt : units - 1;
  // teams past the last row (the last workgroup's) clamp to it and store
  // nothing
  int64_t row0 = team * R;
  int64_t skip = 0;
  if (row0 + R > a.M) {
    skip = row0 + R - a.M;
    row0 = a.M - R;
  }
  // activation loads first, then the first rows' weight loads; what needs
  // the activation (its quantization) waits only for it
  typename F::XRaw xr[1];                 // fp32 values (XF)
  typename F::Act act;
  if constexpr (XF) F::load_x(xr[0], a.x, u);
  else F::issue_act(act, a.y, u);
  __builtin_amdgcn_sched_barrier(0);
  const typename F::Lane L = F::lane(u);
  typename F::Wt w[R];
  const uint8_t* base = a.W + row0 * a.row_bytes;
  const uint32_t rb = static_cast<uint32_t>(a.row_bytes);
#pragma unroll
  for (int r = 0; r < FIRST; ++r) {
    F::load_wt(w[r], base, static_cast<uint32_t>(r) * rb, L);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (XF) F::quant_x(act, xr[0]);
  else F::finish_act(act);
  if (!active) F::zero_act(act);
  float pt[1][R];
  static_for<0, R>([&](auto rc) QMV_INLINE {
    constexpr int r = decltype(rc)::value;
    typename F::Dec dec;
    F::decode(w[r], dec, L);
    pt[0][r] = F::col_dot(dec, act);
    // row r's arithmetic stays ahead of the next issue
    if constexpr (DEPTH > 0) __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEPTH > 0 && r + DEPTH < R) {
      F::load_wt(w[r + DEPTH], base, static_cast<uint32_t>(r + DEPTH) * rb, L);
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  // the team reduction of rows_body: within each wave, then the waves'
  // partials summed in wave order
  team_reduce<kWave, 1, R>(pt, lane);
  using RM = ReduceMap<kWave, R>;
  if (RM::representative(lane)) {
#pragma unroll
    for (int pos = 0; pos < RM::kPerLane; ++pos) red[wave * R + RM::index(lane, pos)] = pt[0][pos];
  }
  __syncthreads();
  if (lt < R && lt >= skip) {
    const int wave0 = team_local * tw;
    float v = 0.0f;
    for (int k = 0; k < tw; ++k) v += red[(wave0 + k) * R + lt];
    if (a.up_scale) v *= a.up_scale[0];
    if (a.up_bias) v += a.up_bias[row0 + lt];
    a.out[row0 + lt] = v;
  }
}

// Columns one rows_body call takes. Where the activation slices of all NC
// columns and the rows in flight exceed the registers, the kernels take the
// columns in two halves (measured spills at 256 registers: Q6_K, 24
// activation words per column, gate/up at 8 columns and in expert blocks
// from 6; Q6_K expert blocks and chunked fp32 rows at 8; the fp32 Q4_K
// whole-chunk expert blocks at 8 with a gate or with two row slots).
template <class F, int G, bool XF, bool ID, bool KLOOP, int P>
constexpr int max_cols_per_call() {
  if (F::kType == 14) {
    if (ID) return G == 2 ? 5 : 7;
    return (G == 2 || (XF && KLOOP)) ? 7 : kMaxCols;
  }
  if (F::kType == 12 && F::kUnitsPerBlock == 4 && ID && XF && (G == 2 || P == 2)) return 7;
  return kMaxCols;
}

// Plain / fused kernel: columns 0..NC-1 of y; a team owns PASSES * R * P
// rows, taken R * P at a time (KLOOP: rows longer than the team, in chunks).
template <class F, int NC, int R, int P, int G, bool XF, int PASSES, int DEPTH = 0, bool KLOOP = false>
__global__ void __launch_bounds__(kLaunchBound) mmvq_rows_kernel(RowArgs a) {
  Cols cols;
  cols.n = NC;
#pragma unroll
  for (int j = 0; j < kMaxCols; ++j) { cols.tok[j] = j; cols.slots[j] = 0; }
  constexpr int V = pow2ceil(NC * R * P);
  __shared__ RedLds<G, V> red;
  constexpr int MC = max_cols_per_call<F, G, XF, false, KLOOP, P>();
  if constexpr (NC <= MC) {
    rows_body<F, NC, R, P, G, false, XF, V, PASSES, DEPTH, KLOOP>(a, cols, a.W, a.Wg, red);
  } else {
    // two halves of the columns; the second re-reads the team's rows (from
    // cache) with its columns' activations and outputs
    constexpr int N0 = (NC + 1) / 2;
    rows_body<F, N0, R, P, G, false, XF, V, PASSES, DEPTH, KLOOP>(a, cols, a.W, a.Wg, red);
    __syncthreads();       // the first half's LDS readers are done
    RowArgs a2 = a;
    if constexpr (XF) a2.x += N0 * a.ldx;
    else a2.y += N0 * a.ycol_bytes;
    a2.out += N0 * a.M;
    rows_body<F, NC - N0, R, P, G, false, XF, V, PASSES, DEPTH, KLOOP>(a2, cols, a2.W, a2.Wg, red);
  }
}

// Expert-indexed kernel: blockIdx.y = expert. The token list is the same for
// every thread of the block (ids are read with uniform addresses). The slice
// blockIdx.y == n_experts, when launched, is the shared expert: every token,
// its own matrices and output, the GLU without scales or biases.
// Rows per pass of an expert block with NC tokens: what the register budget
// allows for NC columns, at most RB; the team owns RB * P rows and takes them
// in RB / id_rows passes.
template <class F, int NC, int RB, int G, bool XF>
constexpr int id_rows() {
  return id_rows_n<F>(NC, RB, G, XF);
}

template <class F, int RB, int P, int G, bool XF>
constexpr int id_lds_values() {
  int v = 1;
  for (int nc = 1; nc <= kMaxCols; ++nc) {
    const int w = pow2ceil(nc * id_rows_n<F>(nc, RB, G, XF) * P);
    if (w > v) v = w;
  }
  return v;
}

// KLOOP: rows longer than the team (RB = 1: one row per pass).
template <class F, int RB, int P, int G, bool XF, bool KLOOP = false>
__global__ void __launch_bounds__(kLaunchBound) mmvq_id_kernel(RowArgs a) {
  static_assert(!KLOOP || (RB == 1 && P == 1), "chunked expert rows: one row, one slot");
  const int e = blockIdx.y;
  const bool shared = e == a.n_experts;
  if (shared) {
    a.W = a.Ws_up;
    a.Wg = a.Ws_gate;
    a.out = a.shared_out;
    a.top_k = 1;
    a.expert_stride = 0;
    a.up_bias = a.gate_bias = a.up_scale = a.gate_scale = nullptr;
  }
  // Tokens routed to expert e, compacted with compile-time indices only (a
  // runtime index into a register array would go through scratch memory).
  uint64_t m[kMaxCols];
#pragma unroll
  for (int t = 0; t < kMaxCols; ++t) {
    m[t] = 0;
    if (t < a.n_tokens) {
      if (shared) {
        m[t] = 1;
      } else {
        for (int k = 0; k < a.top_k; ++k)
          if (a.ids[t * a.top_k + k] == e) m[t] |= 1ull << k;
      }
    }
  }
  Cols cols;
  cols.n = 0;
#pragma unroll
  for (int j = 0; j < kMaxCols; ++j) { cols.tok[j] = 0; cols.slots[j] = 0; }
#pragma unroll
  for (int t = 0; t < kMaxCols; ++t) {
    if (m[t]) {
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j)
        if (j == cols.n) { cols.tok[j] = t; cols.slots[j] = m[t]; }
      ++cols.n;
    }
  }
  if (cols.n == 0) return;     // uniform: the whole block leaves together
  const int64_t eo = shared ? 0 : static_cast<int64_t>(e) * a.expert_stride;
  const uint8_t* We = a.W + eo;
  const uint8_t* Wge = G == 2 ? a.Wg + eo : nullptr;
  constexpr int VMAX = id_lds_values<F, RB, P, G, XF>();
  __shared__ RedLds<G, VMAX> red;
  auto run = [&](auto nc, const Cols& c) QMV_INLINE {
    constexpr int NC = decltype(nc)::value;
    constexpr int R = id_rows<F, NC, RB, G, XF>();
    rows_body<F, NC, R, P, G, true, XF, VMAX, RB / R, 0, KLOOP>(a, c, We, Wge, red);
  };
  // more tokens than the registers hold at once: two halves, the second
  // re-reading the block's rows (from cache) for the other tokens
  constexpr int MC = max_cols_per_call<F, G, XF, true, KLOOP, P>();
  auto run_split = [&](auto nc) QMV_INLINE {
    constexpr int NC = decltype(nc)::value;
    if constexpr (NC <= MC) {
      run(nc, cols);
    } else {
      constexpr int N0 = (NC + 1) / 2;
      run(Idx<N0>{}, cols);
      __syncthreads();     // the first half's LDS readers are done
      Cols c2;
      c2.n = NC - N0;
#pragma unroll
      for (int j = 0; j < kMaxCols; ++j) {
        c2.tok[j] = j + N0 < kMaxCols ? cols.tok[j + N0 < kMaxCols ? j + N0 : 0] : 0;
        c2.slots[j] = j + N0 < kMaxCols ? cols.slots[j + N0 < kMaxCols ? j + N0 : 0] : 0;
      }
      run(Idx<NC - N0>{}, c2);
    }
  };
  switch (cols.n) {
#define QMV_ID_CASE(NC) run_split(Idx<NC>{})
    case 1: QMV_ID_CASE(1); break;
    case 2: QMV_ID_CASE(2); break;
    case 3: QMV_ID_CASE(3); break;
    case 4: QMV_ID_CASE(4); break;
    case 5: QMV_ID_CASE(5); break;
    case 6: QMV_ID_CASE(6); break;
    case 7: QMV_ID_CASE(7); break;
    default: QMV_ID_CASE(8); break;
#undef QMV_ID_CASE
  }
}

// Test support: integer dots of every (column, row, block), one thread per
// (column, row, block), through the same load/decode routines.
template <class F>
__global__ void __launch_bounds__(256) mmvq_block_dots_kernel(const uint8_t* W, const uint8_t* y,
                                                              int32_t* dots, int64_t M, int64_t nblocks,
                                                              int64_t row_bytes, int64_t ycol_bytes,
                                                              int64_t n) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // 256-lane blocks
  if (gid >= n * M * nblocks) return;
  const int64_t b = gid % nblocks;
  const int64_t r = (gid / nblocks) % M;
  const int64_t j = gid / (nblocks * M);
  int acc[F::kDotsPerBlock];
#pragma unroll
  for (int k = 0; k < F::kDotsPerBlock; ++k) acc[k] = 0;
  for (int q = 0; q < F::kUnitsPerBlock; ++q) {
    const int u = static_cast<int>(b) * F::kUnitsPerBlock + q;
    const typename F::Lane L = F::lane(u);
    typename F::Wt w;
    F::load_wt(w, W + r * row_bytes, 0u, L);
    typename F::Dec dec;
    F::decode(w, dec, L);
    F::int_dots(dec, y + j * ycol_bytes, u, acc);
  }
  int32_t* o = dots + gid * F::kDotsPerBlock;
#pragma unroll
  for (int k = 0; k < F::kDotsPerBlock; ++k) o[k] = acc[k];
}

}  // namespace qmv
