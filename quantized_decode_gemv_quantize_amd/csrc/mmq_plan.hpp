// mmq_plan.hpp - addressing of the many-column (MFMA) kernel: argument
// block, K split, operand pointers and the loads of one super-block. Pure
// pointer arithmetic and loads, shared by the kernel and the host model of
// its memory accesses.
#pragma once

#include "common.hpp"
#include "formats.hpp"

namespace qmv {

struct MmqArgs {
  const uint8_t* W;
  const uint8_t* y;          // q8_1 columns
  float* out;                // out[c*M + r]
  const float* up_bias;      // epilogue without a gate: out*up_scale[0] + up_bias[r]
  const float* up_scale;
  int64_t M;
  int64_t row_bytes;
  int64_t ycol_bytes;
  int n;                     // columns
  int nsb;                   // super-blocks per row
};

// First super-block of wave w's share of the K range when nw waves split it
// (w = 0..nw).
__host__ __device__ __forceinline__ int mmq_sb_begin(int nsb, int w, int nw) { return (nsb * w) / nw; }

// Staging loads of super-block sb: every load is a 16-byte piece of a
// contiguous run, so a wave's loads cover whole cache lines. A: the 16 rows'
// 144-byte super-blocks of each row tile, 144 pieces per tile (row tile
// k / 144, row (k % 144) / 9); B: the 16 columns' 8 q8_1 blocks of each column
// tile, a 288-byte run per column, 288 pieces per tile (column tile k / 288,
// column (k % 288) / 18). Lane L takes pieces L, L + 64, ...; pieces past the
// end are not loaded. Piece k lands at byte 16k of the wave's A or B tiles in
// LDS, which the kernel reads the MFMA operands from.
constexpr int kMmqAPieces = 144, kMmqBPieces = 288;
template <int RT>
constexpr int mmq_a_slots() { return (kMmqAPieces * RT + kWave - 1) / kWave; }
template <int CT>
constexpr int mmq_b_slots() { return (kMmqBPieces * CT + kWave - 1) / kWave; }

template <int RT, int CT>
struct MmqStage {
  u32x4 a[mmq_a_slots<RT>()];
  u32x4 b[mmq_b_slots<CT>()];
};

// Piece offsets of a lane, fixed for the whole K range: the byte offset of
// each piece from the tile's first row (A) or first column (B) at super-block
// 0. Rows past M - 1 and columns past n - 1 are clamped to the last one
// (they are read and computed, never stored; each output column depends only
// on its own). Offsets are 32-bit: a tile spans at most 32 rows or columns.
template <int RT, int CT>
struct MmqOffsets {
  uint32_t a[mmq_a_slots<RT>()];
  uint32_t b[mmq_b_slots<CT>()];
};

template <int RT, int CT>
__host__ __device__ __forceinline__ void mmq_offsets(const MmqArgs& a, int64_t row_base, int col_base, int lane,
                                                     MmqOffsets<RT, CT>& o) {
#pragma unroll
  for (int j = 0; j < mmq_a_slots<RT>(); ++j) {
    const int k = lane + kWave * j, kk = k % kMmqAPieces;
    int64_t r = row_base + 16 * (k / kMmqAPieces) + kk / 9;
    r = r < a.M ? r : a.M - 1;
    o.a[j] = static_cast<uint32_t>((r - row_base) * a.row_bytes + 16 * (kk % 9));
  }
#pragma unroll
  for (int j = 0; j < mmq_b_slots<CT>(); ++j) {
    const int k = lane + kWave * j, kk = k % kMmqBPieces;
    int c = col_base + 16 * (k / kMmqBPieces) + kk / 18;
    c = c < a.n ? c : a.n - 1;
    o.b[j] = static_cast<uint32_t>(static_cast<int64_t>(c - col_base) * a.ycol_bytes + 16 * (kk % 18));
  }
}

// The staging loads of super-block sb: a wave-uniform base per operand plus
// the lane's offsets; pieces past the end (k >= 144*RT or 288*CT) are not
// loaded.
template <int RT, int CT>
__device__ __forceinline__ void mmq_stage_load(const MmqArgs& a, int64_t row_base, int col_base, int lane, int sb,
                                               const MmqOffsets<RT, CT>& o, MmqStage<RT, CT>& st) {
  const uint8_t* wb = a.W + (row_base * a.row_bytes + static_cast<int64_t>(sb) * 144);
  const uint8_t* yb = a.y + (static_cast<int64_t>(col_base) * a.ycol_bytes + static_cast<int64_t>(sb) * 288);
#pragma unroll
  for (int j = 0; j < mmq_a_slots<RT>(); ++j)
    if (lane + kWave * j < kMmqAPieces * RT) st.a[j] = ld_a16_x4(wb + o.a[j]);
#pragma unroll
  for (int j = 0; j < mmq_b_slots<CT>(); ++j)
    if (lane + kWave * j < kMmqBPieces * CT) st.b[j] = ld_a16_x4(yb + o.b[j]);
}

// Output of partial value v (0 .. RT*CT*4-1) of a lane with k-slice q and
// column r16 in the result layout: tile (rt, ct), row 4q + i of the tile.
template <int RT, int CT>
__host__ __device__ __forceinline__ void mmq_store_pos(int v, int q, int r16, int64_t row_base, int col_base,
                                                       int64_t& r, int& c) {
  const int rt = v / (CT * 4), ct = (v / 4) % CT, i = v % 4;
  r = row_base + 16 * rt + 4 * q + i;
  c = col_base + 16 * ct + r16;
}

}  // namespace qmv
