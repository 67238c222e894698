// mmq_plan.hpp - addressing of the many-column (MFMA) kernel: argument
// block, workgroup-to-tile mapping, K split, operand pointers and the loads
// of one staging step. Pure pointer arithmetic and loads, shared by the
// kernel and the host model of its memory accesses.
#pragma once

#include "common.hpp"
#include "formats.hpp"

namespace qmv {

struct MmqArgs {
  const uint8_t* W;          // up (or plain) weights
  const uint8_t* Wg;         // gate weights (gate/up form), same layout; NULL without a gate
  const uint8_t* y;          // q8_1 columns
  const float* x;            // fp32 columns instead (the fused form), column stride ldx; NULL: y
  int64_t ldx;
  float* out;                // out[c*M + r]
  // epilogue: up = up*up_scale[0] + up_bias[r], the same for the gate, then
  // glu(glu_op, gate, up, glu_limit) in the gate/up form; NULL pointers are
  // skipped
  const float* up_bias;
  const float* up_scale;
  const float* gate_bias;
  const float* gate_scale;
  int glu_op;
  float glu_limit;
  int64_t M;
  int64_t row_bytes;
  int64_t ycol_bytes;
  int n;                     // columns
  int nsb;                   // staging steps per row (256 weights each)
  int gx, gy;                // row tiles and column tiles of the grid
};

// Staging geometry of a weight format: a staging step covers 256 weights of
// a row (the 8 q8_1 blocks of one step of the activation), kStride bytes of
// the row, staged with kRowPieces loads per row into a kRowLds-byte row
// image in LDS. Formats whose steps are 16-byte multiples (Q4_K 144, Q5_K
// 176, Q4_0 8 x 18 = 144, Q4_1 8 x 20 = 160, Q5_0 8 x 22 = 176, Q5_1
// 8 x 24 = 192, Q8_0 8 x 34 = 272 bytes) stage them as 16-byte pieces at
// 16-byte aligned addresses; step byte y sits at image byte y.
template <class F> struct MmqGeom;
template <int STRIDE>
struct MmqGeomAligned {
  static constexpr int kStride = STRIDE, kRowPieces = STRIDE / 16, kRowLds = STRIDE;
  __host__ __device__ static int image_base(int64_t, int) { return 0; }
  __host__ __device__ static int piece_lds(int64_t, int, int pc) { return 16 * pc; }
  __host__ __device__ static bool piece_short(int) { return false; }
  __host__ __device__ static int64_t piece_src(int64_t row_off, int sb, int pc) {
    return row_off + static_cast<int64_t>(sb) * STRIDE + 16 * pc;
  }
};
template <> struct MmqGeom<Q4K> : MmqGeomAligned<144> {};
template <> struct MmqGeom<Q40> : MmqGeomAligned<144> {};
template <> struct MmqGeom<Q80> : MmqGeomAligned<272> {};
template <> struct MmqGeom<Q41> : MmqGeomAligned<160> {};
template <> struct MmqGeom<Q50> : MmqGeomAligned<176> {};
template <> struct MmqGeom<Q51> : MmqGeomAligned<192> {};
template <> struct MmqGeom<Q5K> : MmqGeomAligned<176> {};
// Q6_K super-blocks (210 bytes) are only 2-byte aligned. As in the row
// kernels every load stays inside its super-block: 13 sixteen-byte runs at
// the first dword-aligned byte s' = s + delta (delta = 0 or 2) plus the one
// 16-bit word the runs miss (the last one when delta = 0, the first one when
// delta = 2). The image keeps 16 bytes of headroom so the runs land 16-byte
// aligned: super-block byte y sits at image byte 16 + y - delta.
template <> struct MmqGeom<Q6K> {
  static constexpr int kStride = 210, kRowPieces = 14, kRowLds = 240;
  __host__ __device__ static int delta(int64_t row_off, int sb) {
    return static_cast<int>((row_off + static_cast<int64_t>(sb) * 210) & 2);
  }
  __host__ __device__ static int image_base(int64_t row_off, int sb) { return 16 - delta(row_off, sb); }
  __host__ __device__ static bool piece_short(int pc) { return pc == 13; }
  __host__ __device__ static int piece_lds(int64_t row_off, int sb, int pc) {
    return pc < 13 ? 16 + 16 * pc : (delta(row_off, sb) ? 14 : 224);
  }
  __host__ __device__ static int64_t piece_src(int64_t row_off, int sb, int pc) {
    const int64_t s = row_off + static_cast<int64_t>(sb) * 210;
    const int d = delta(row_off, sb);
    return pc < 13 ? s + d + 16 * pc : (d ? s : s + 208);
  }
};

// Workgroup w -> tile (bx: row tile, by: column tile). Workgroups go to the
// 8 XCDs round-robin (w mod 8), and each XCD has its own L2; the mapping
// gives each XCD a contiguous range of tiles in row-tile-major order, so the
// column tiles of one row tile run on the same XCD one after another and
// re-read the row tile's weights from that L2 rather than from HBM. A
// bijection of [0, gx*gy) for any grid size.
constexpr int kXcds = 8;
__host__ __device__ __forceinline__ void mmq_tile_of(int64_t w, int gx, int gy, int64_t& bx, int& by) {
  const int64_t N = static_cast<int64_t>(gx) * gy;
  const int64_t x = w % kXcds, j = w / kXcds;
  const int64_t per = N / kXcds, extra = N % kXcds;
  const int64_t t = x * per + (x < extra ? x : extra) + j;
  bx = t / gy;
  by = static_cast<int>(t - bx * gy);
}

// First staging step of wave w's share of the K range when nw waves split
// it (w = 0..nw).
__host__ __device__ __forceinline__ int mmq_sb_begin(int nsb, int w, int nw) { return (nsb * w) / nw; }

// Staging loads of step sb: every load is a 16-byte piece of a contiguous
// run (or Q6_K's one 16-bit word per row), so a wave's loads cover whole
// cache lines. A: kRowPieces loads of each of the 16 rows of each row tile
// (row tile k / (16*kRowPieces), row (k % (16*kRowPieces)) / kRowPieces);
// B: the 16 columns' 8 q8_1 blocks of each column tile, a 288-byte run per
// column, 288 pieces per tile (column tile k / 288, column (k % 288) / 18).
// Lane L takes loads L, L + 64, ...; loads past the end are not issued.
// A piece lands in its row's image in LDS (piece_lds), B piece k at byte 16k
// of the B tiles.
constexpr int kMmqBPieces = 288;
template <class F>
constexpr int mmq_a_pieces() { return 16 * MmqGeom<F>::kRowPieces; }
template <class F, int RT>
constexpr int mmq_a_slots() { return (mmq_a_pieces<F>() * RT + kWave - 1) / kWave; }
template <int CT>
constexpr int mmq_b_slots() { return (kMmqBPieces * CT + kWave - 1) / kWave; }

// The fused form (fp32 columns) stages the step's activations raw: each of
// the 16*CT*8 (column, block) pairs of the step is one lane's 32 values
// (pair k = lane + 64*j: column tile k / 128, column (k % 128) / 8, block
// k % 8), quantized by that lane before they go to LDS.
template <int CT>
constexpr int mmq_x_slots() { return 16 * 8 * CT / kWave; }
template <int CT, bool XF> struct MmqBStage { u32x4 b[mmq_b_slots<CT>()]; };
template <int CT> struct MmqBStage<CT, true> { u32x4 x[mmq_x_slots<CT>()][8]; };

template <class F, int RT, int CT, int G, bool XF = false>
struct MmqStage : MmqBStage<CT, XF> {
  u32x4 a[G][mmq_a_slots<F, RT>()];   // [0] up (or plain) rows, [1] gate rows
};

// Column and block of fused-form pair slot j of a lane (column within the
// workgroup's CT tiles; clamped to n - 1 like the q8_1 columns).
__host__ __device__ __forceinline__ void mmq_x_pair(int lane, int j, int col_base, int n, int& col, int& blk,
                                                    int& c) {
  const int k = lane + kWave * j;
  col = 16 * (k / 128) + (k % 128) / 8;
  blk = k % 8;
  c = col_base + col < n ? col_base + col : n - 1;
}

// Load slots of a lane, fixed for the whole K range: for A the byte offset
// of the slot's row from the tile's first row, its row within the tile
// (0..16*RT-1) and its piece within the row; for B the offset of the piece
// from the tile's first column. Rows past M - 1 and columns past n - 1 are
// clamped to the last one (they are read and computed, never stored; each
// output depends only on its own row and column). Offsets are 32-bit: a
// tile spans at most 32 rows or columns.
template <class F, int RT, int CT>
struct MmqOffsets {
  uint32_t a[mmq_a_slots<F, RT>()];
  uint8_t arow[mmq_a_slots<F, RT>()];
  uint8_t apc[mmq_a_slots<F, RT>()];
  uint32_t b[mmq_b_slots<CT>()];
};

template <class F, int RT, int CT>
__host__ __device__ __forceinline__ void mmq_offsets(const MmqArgs& a, int64_t row_base, int col_base, int lane,
                                                     MmqOffsets<F, RT, CT>& o) {
  constexpr int RP = MmqGeom<F>::kRowPieces;
#pragma unroll
  for (int j = 0; j < mmq_a_slots<F, RT>(); ++j) {
    const int k = lane + kWave * j;
    const int row = k / RP < 16 * RT ? k / RP : 16 * RT - 1;     // slots past the end: any valid row
    int64_t r = row_base + row;
    r = r < a.M ? r : a.M - 1;
    o.a[j] = static_cast<uint32_t>((r - row_base) * a.row_bytes);
    o.arow[j] = static_cast<uint8_t>(row);
    o.apc[j] = static_cast<uint8_t>(k % RP);
  }
#pragma unroll
  for (int j = 0; j < mmq_b_slots<CT>(); ++j) {
    const int k = lane + kWave * j, kk = k % kMmqBPieces;
    int c = col_base + 16 * (k / kMmqBPieces) + kk / 18;
    c = c < a.n ? c : a.n - 1;
    o.b[j] = static_cast<uint32_t>(static_cast<int64_t>(c - col_base) * a.ycol_bytes + 16 * (kk % 18));
  }
}

// The staging loads of step sb; loads past the end (slot k >= the tile's
// loads) are not issued. The gate rows (G = 2) sit at the same offsets of
// Wg as the up rows of W. Weights (A) and activations (B) separately, so the
// fp32 form can have the next weights in flight while it quantizes.
template <class F, int RT, int CT, int G, bool XF>
__device__ __forceinline__ void mmq_stage_load_a(const MmqArgs& a, int64_t row_base, int lane, int sb,
                                                 const MmqOffsets<F, RT, CT>& o, MmqStage<F, RT, CT, G, XF>& st) {
  using Gm = MmqGeom<F>;
  const int64_t tile_off = row_base * a.row_bytes;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint8_t* W = g == 0 ? a.W : a.Wg;
#pragma unroll
    for (int j = 0; j < mmq_a_slots<F, RT>(); ++j) {
      if (lane + kWave * j < mmq_a_pieces<F>() * RT) {
        const uint8_t* src = W + Gm::piece_src(tile_off + o.a[j], sb, o.apc[j]);
        if (Gm::piece_short(o.apc[j])) st.a[g][j].x = ld_u16(src);
        else if constexpr (MmqGeom<F>::kStride % 16 == 0) st.a[g][j] = ld_a16_x4(src);
        else st.a[g][j] = ld_x4(src);
      }
    }
  }
}

// fp32 columns: the 32 values of pair slot j of a lane at step sb
template <class F, int RT, int CT, int G>
__device__ __forceinline__ void mmq_stage_load_x(const MmqArgs& a, int col_base, int lane, int sb, int j,
                                                 MmqStage<F, RT, CT, G, true>& st) {
  int col, blk, c;
  mmq_x_pair(lane, j, col_base, a.n, col, blk, c);
  const float* p = a.x + (static_cast<int64_t>(c) * a.ldx + static_cast<int64_t>(sb) * 256 + 32 * blk);
#pragma unroll
  for (int k = 0; k < 8; ++k) st.x[j][k] = ld_x4(reinterpret_cast<const uint8_t*>(p + 4 * k));
}

template <class F, int RT, int CT, int G, bool XF>
__device__ __forceinline__ void mmq_stage_load_b(const MmqArgs& a, int col_base, int lane, int sb,
                                                 const MmqOffsets<F, RT, CT>& o, MmqStage<F, RT, CT, G, XF>& st) {
  if constexpr (XF) {
#pragma unroll
    for (int j = 0; j < mmq_x_slots<CT>(); ++j) mmq_stage_load_x<F, RT, CT, G>(a, col_base, lane, sb, j, st);
  } else {
    const uint8_t* yb = a.y + (static_cast<int64_t>(col_base) * a.ycol_bytes + static_cast<int64_t>(sb) * 288);
#pragma unroll
    for (int j = 0; j < mmq_b_slots<CT>(); ++j)
      if (lane + kWave * j < kMmqBPieces * CT) st.b[j] = ld_a16_x4(yb + o.b[j]);
  }
}

template <class F, int RT, int CT, int G, bool XF = false>
__device__ __forceinline__ void mmq_stage_load(const MmqArgs& a, int64_t row_base, int col_base, int lane, int sb,
                                               const MmqOffsets<F, RT, CT>& o, MmqStage<F, RT, CT, G, XF>& st) {
  mmq_stage_load_a<F, RT, CT, G, XF>(a, row_base, lane, sb, o, st);
  mmq_stage_load_b<F, RT, CT, G, XF>(a, col_base, lane, sb, o, st);
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
