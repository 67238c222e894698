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

constexpr int kMmqWaves = 4;

// First super-block of wave w's share of the K range (w = 0..kMmqWaves).
__host__ __device__ __forceinline__ int mmq_sb_begin(int nsb, int w) { return (nsb * w) / kMmqWaves; }

// Operand pointers of one lane: A rows row_base + 16*rt + r16 (clamped to the
// matrix: rows past M are loaded but never stored) and B columns
// col_base + 16*ct + r16 (clamped: columns past n contribute zero).
template <int RT, int CT>
__device__ __forceinline__ void mmq_pointers(const MmqArgs& a, int64_t row_base, int col_base, int r16,
                                             const uint8_t* (&arow)[RT], const uint8_t* (&bcol)[CT],
                                             bool (&bvalid)[CT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t r = row_base + 16 * rt + r16;
    r = r < a.M ? r : a.M - 1;
    arow[rt] = a.W + r * a.row_bytes;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int c = col_base + 16 * ct + r16;
    bvalid[ct] = c < a.n;
    bcol[ct] = a.y + static_cast<int64_t>(bvalid[ct] ? c : a.n - 1) * a.ycol_bytes;
  }
}

// Loads of super-block sb for a lane of k-slice q: the row headers, the
// 8 code bytes of each 64-element chunk at offset 8q (low nibbles feed
// sub-block 2c, high nibbles 2c+1), and the q8_1 codes 8q..8q+7 and fp16 d
// of the 8 blocks of each column.
template <int RT, int CT>
struct MmqQ4KLoads {
  u32x4 hdr[RT];
  u32x2 qs[RT][4];
  u32x2 yq[CT][8];
  uint32_t yd[CT][8];
};

template <int RT, int CT>
__device__ __forceinline__ void mmq_q4k_load(const uint8_t* const (&arow)[RT], const uint8_t* const (&bcol)[CT],
                                             int sb, int q, MmqQ4KLoads<RT, CT>& ld) {
  const int64_t boff = static_cast<int64_t>(sb) * Q4K::kBlockBytes;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    ld.hdr[rt] = ld_x4(arow[rt] + boff);
#pragma unroll
    for (int c = 0; c < 4; ++c) ld.qs[rt][c] = ld_x2(arow[rt] + (boff + 16 + 32 * c + 8 * q));
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint8_t* b = bcol[ct] + static_cast<int64_t>(8 * sb + t) * kQ8Bytes;
      ld.yq[ct][t] = ld_x2(b + 4 + 8 * q);
      ld.yd[ct][t] = ld_u16(b);
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
