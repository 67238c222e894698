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
// 144-byte super-blocks of each row tile (144 pieces, row = k / 9); B: the
// 16 columns' 8 q8_1 blocks of each column tile (a 288-byte run per column,
// 288 pieces, column = k / 18). Lane L takes pieces L, L + 64, ...; pieces
// past the end are not loaded. The kernel stores them to LDS and reads the
// MFMA operands from there.
constexpr int kMmqAPieces = 144, kMmqBPieces = 288;
constexpr int kMmqAPerLane = (kMmqAPieces + kWave - 1) / kWave;   // 3
constexpr int kMmqBPerLane = (kMmqBPieces + kWave - 1) / kWave;   // 5

template <int RT, int CT>
struct MmqStage {
  u32x4 a[RT][kMmqAPerLane];
  u32x4 b[CT][kMmqBPerLane];
};

// Piece pointers of a lane: rows of the row tiles and columns of the column
// tiles, clamped to the matrix and to n (clamped rows and columns are read
// and computed, never stored; each output column depends only on its own).
template <int RT, int CT>
__device__ __forceinline__ void mmq_stage_load(const MmqArgs& a, int64_t row_base, int col_base, int lane, int sb,
                                               MmqStage<RT, CT>& st) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < kMmqAPerLane; ++j) {
      const int k = lane + kWave * j;
      if (k < kMmqAPieces) {
        int64_t r = row_base + 16 * rt + k / 9;
        r = r < a.M ? r : a.M - 1;
        st.a[rt][j] = ld_a16_x4(a.W + (r * a.row_bytes + static_cast<int64_t>(sb) * 144 + 16 * (k % 9)));
      }
    }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int j = 0; j < kMmqBPerLane; ++j) {
      const int k = lane + kWave * j;
      if (k < kMmqBPieces) {
        int c = col_base + 16 * ct + k / 18;
        c = c < a.n ? c : a.n - 1;
        st.b[ct][j] = ld_a16_x4(a.y + (static_cast<int64_t>(c) * a.ycol_bytes + static_cast<int64_t>(sb) * 288 +
                                       16 * (k % 18)));
      }
    }
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
