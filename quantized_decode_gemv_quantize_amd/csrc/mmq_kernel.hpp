// mmq_kernel.hpp - the many-column path (6 or more activation columns) for
// Q4_K weights: int8 matrix-core (MFMA) products of 16x16 tiles.
//
// Citations: [MMVQ §X] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时
// 一条量化权重如何被 dp4a 逐块点积", section X.
//
// Beyond a handful of columns the per-column integer dots of the mat-vec
// kernels cost more than the weight stream [MMVQ §多个 token 时, §分派]; here
// the weights are decoded once into MFMA operands and reused across 16-column
// tiles, and the integer dots of every (row, column, 32-element sub-block) come
// from v_mfma_i32_16x16x32_i8: A = 16 rows x 32 codes of one sub-block, B = the
// matching q8_1 block of 16 columns. The block scales are those of the mat-vec
// [MMVQ §一次 vec_dot 的解剖], summed in another order:
//   out[r][c] += d[r] * sum_t sc_t[r]*C_t[r][c] * d8_t[c]
//              - dmin[r] * sum_t m_t[r] * (d8_t[c]*S_t[c])
// with C_t the int32 tile of sub-block t and S_t[c] the sum of the q8_1 codes
// of column c in block t. sc_t*C_t is an exact integer (below 2^22), so each
// sub-block costs one fp32 multiply-add per output; d is applied once per
// super-block, and the min term, a contraction over the 8 sub-blocks of an
// 8-long column of -dmin*m_t by an 8-long row of d8_t*S_t, is two fp32 MFMAs
// (v_mfma_f32_16x16x4_f32, even and odd t) per tile and super-block.
//
// A workgroup owns RT x CT tiles (16 rows x 16 columns each); its NW waves
// split the K range (super-blocks) and their fp32 partials are summed through
// LDS in a fixed order. MFMA lane layouts (checked on the device):
//   i8 A: lane l holds row l%16, codes k = 8*(l/16) .. +7
//   i8 B: lane l holds column l%16, codes k = 8*(l/16) .. +7
//   f32 A: lane l holds row l%16, k = l/16; f32 B: column l%16, k = l/16
//   D (both): lane l holds rows 4*(l/16) .. +3 of column l%16
#pragma once

#include "common.hpp"
#include "formats.hpp"
#include "mmq_plan.hpp"

namespace qmv {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));


__device__ __forceinline__ long pack2(uint32_t lo, uint32_t hi) {
  return static_cast<long>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// LDS of one wave: the staged super-block tiles and the row factors.
template <int RT, int CT>
struct MmqWaveLds {
  uint8_t a[RT][16][144];          // 16 rows' super-blocks
  uint8_t b[CT][16][288];          // 16 columns' 8 q8_1 blocks
  uint8_t sc[RT][4][16][2];        // sc_t of row, t = 2c + h at [c][row][h]
  float d[RT][16];                 // d of row
};

// LDS bytes of a workgroup (the staging tiles of all waves; the reduction
// reuses them), and the shapes that fit one compute unit's 160 KB.
template <int RT, int CT, int NW>
constexpr size_t mmq_lds_bytes() {
  const size_t stage = sizeof(MmqWaveLds<RT, CT>) * NW, red = sizeof(float) * NW * RT * CT * 4 * kWave;
  return stage > red ? stage : red;
}
template <int RT, int CT, int NW>
constexpr bool mmq_fits() { return mmq_lds_bytes<RT, CT, NW>() <= 160 * 1024; }

template <int RT, int CT, int NW>
__global__ void __launch_bounds__(NW * kWave, 8 / NW) mmq_q4k_kernel(MmqArgs a) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (16 * RT);
  const int col_base = static_cast<int>(blockIdx.y) * (16 * CT);
  const int sb0 = mmq_sb_begin(a.nsb, wave, NW), sb1 = mmq_sb_begin(a.nsb, wave + 1, NW);
  const Q4K::Lane L = Q4K::lane(2 * q);       // scale unpack of chunk q (sub-blocks 2q, 2q+1)

  // the staging tiles of the NW waves; after the K loop the same LDS holds
  // the partial sums of the reduction
  constexpr int NV = RT * CT * 4;
  __shared__ __align__(16) uint8_t smem[mmq_lds_bytes<RT, CT, NW>()];
  MmqWaveLds<RT, CT>& lds = reinterpret_cast<MmqWaveLds<RT, CT>*>(smem)[wave];
  float acc[RT][CT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][ct][i] = 0.0f;

  // staged pieces -> LDS: piece k at byte 16k of the A or B tiles
  auto store_stage = [&](const MmqStage<RT, CT>& st) {
    uint8_t* la = &lds.a[0][0][0];
    uint8_t* lb = &lds.b[0][0][0];
#pragma unroll
    for (int j = 0; j < mmq_a_slots<RT>(); ++j) {
      const int k = lane + kWave * j;
      if (k < kMmqAPieces * RT) *reinterpret_cast<u32x4*>(la + 16 * k) = st.a[j];
    }
#pragma unroll
    for (int j = 0; j < mmq_b_slots<CT>(); ++j) {
      const int k = lane + kWave * j;
      if (k < kMmqBPieces * CT) *reinterpret_cast<u32x4*>(lb + 16 * k) = st.b[j];
    }
  };

  // LDS accesses of one wave complete in order; the waits make the data
  // written by other lanes of the wave visible to the reads that follow
  auto lds_fence = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };

  // one super-block from LDS. Lane (r16, q) unpacks sub-blocks 2q and 2q+1
  // of row r16: the f32 A operand of the min term (k = q stands for t = 2q in
  // the even product, t = 2q+1 in the odd one) and the scales, which the D
  // layout reads back per chunk for rows 4q..4q+3.
  auto compute = [&]() {
    const long ones = 0x0101010101010101l;
    float am[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const u32x4 hdr = *reinterpret_cast<const u32x4*>(&lds.a[rt][r16][0]);
      uint32_t scp, mp;
      Q4K::chunk_scales(hdr, L, scp, mp);
      *reinterpret_cast<uint16_t*>(&lds.sc[rt][q][r16][0]) = static_cast<uint16_t>(scp & 0xFFFFu);
      lds.d[rt][r16] = h2f(hdr.x);
      const float dmin = h2f(hdr.x >> 16);
      am[rt][0] = -dmin * static_cast<float>(mp & 0xFFu);
      am[rt][1] = -dmin * static_cast<float>((mp >> 8) & 0xFFu);
    }
    lds_fence();

    float accd[RT][CT][4], e[CT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) accd[rt][ct][i] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) e[ct][0] = e[ct][1] = 0.0f;
    // sub-blocks 2c and 2c+1 share the code bytes of chunk c (low and high
    // nibbles); the chunk loop is kept rolled so only one chunk's operands
    // are live
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      u32x2 w[RT], scw[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        w[rt] = *reinterpret_cast<const u32x2*>(&lds.a[rt][r16][16 + 32 * c + 8 * q]);
        scw[rt] = *reinterpret_cast<const u32x2*>(&lds.sc[rt][c][4 * q][0]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * c + h;
        long A[RT];
        int sc[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          A[rt] = pack2((w[rt].x >> (4 * h)) & 0x0F0F0F0Fu, (w[rt].y >> (4 * h)) & 0x0F0F0F0Fu);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[rt][i] = static_cast<int>(((i < 2 ? scw[rt].x : scw[rt].y) >> (8 * (2 * (i & 1) + h))) & 0xFFu);
        }
        // all products of the sub-block first, then their scaling: the
        // multiply-adds of one tile overlap the next tiles' MFMAs
        v4i C[RT][CT];
        float d8[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const uint8_t* blk = &lds.b[ct][r16][36 * t];
          // codes 8q..8q+7 of the block: two dword reads (the block is
          // 36 bytes, so the pair is 8-byte aligned only in odd blocks)
          const uint32_t* cw = reinterpret_cast<const uint32_t*>(blk + 4 + 8 * q);
          const long B = pack2(cw[0], cw[1]);
          d8[ct] = h2f(*reinterpret_cast<const uint16_t*>(blk));
          const v4i zero = {0, 0, 0, 0};
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) C[rt][ct] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], B, zero, 0, 0, 0);
          // code sum of block t of column r16 (every row of the product
          // holds it); lane q keeps blocks 2q and 2q+1 for the min term
          const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, B, zero, 0, 0, 0);
          if (c == q) e[ct][h] = d8[ct] * static_cast<float>(S[0]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              accd[rt][ct][i] = fmaf(static_cast<float>(__mul24(C[rt][ct][i], sc[rt][i])), d8[ct], accd[rt][ct][i]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float4 dv = *reinterpret_cast<const float4*>(&lds.d[rt][4 * q]);
      const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        v4f v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf(dd[i], accd[rt][ct][i], acc[rt][ct][i]);
        v = __builtin_amdgcn_mfma_f32_16x16x4f32(am[rt][0], e[ct][0], v, 0, 0, 0);
        v = __builtin_amdgcn_mfma_f32_16x16x4f32(am[rt][1], e[ct][1], v, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rt][ct][i] = v[i];
      }
    }
  };

  // Pipeline: the staging loads of super-block sb+1 are in flight while sb
  // is computed from LDS. The prefetch is unconditional (past the end it
  // re-reads the last super-block, from cache) so every path has the same
  // loads in flight.
  if (sb0 < sb1) {
    MmqOffsets<RT, CT> off;
    mmq_offsets<RT, CT>(a, row_base, col_base, lane, off);
    MmqStage<RT, CT> st;
    mmq_stage_load<RT, CT>(a, row_base, col_base, lane, sb0, off, st);
    for (int sb = sb0; sb < sb1; ++sb) {
      lds_fence();                 // the previous super-block's reads are done
      store_stage(st);
      const int next = sb + 1 < sb1 ? sb + 1 : sb;
      mmq_stage_load<RT, CT>(a, row_base, col_base, lane, next, off, st);
      __builtin_amdgcn_sched_barrier(0);
      lds_fence();
      compute();
    }
  }

  // ---- sum the waves' partials (in wave order) and store
  __syncthreads();                 // every wave is done with its staging tiles
  float(*red)[NV][kWave] = reinterpret_cast<float(*)[NV][kWave]>(smem);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(rt * CT + ct) * 4 + i][lane] = acc[rt][ct][i];
  __syncthreads();
  for (int v = wave; v < NV; v += NW) {
    float s = red[0][v][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[w][v][lane];
    int64_t r;
    int c;
    mmq_store_pos<RT, CT>(v, q, r16, row_base, col_base, r, c);
    if (r < a.M && c < a.n) {
      float o = s;
      if (a.up_scale) o *= a.up_scale[0];
      if (a.up_bias) o += a.up_bias[r];
      a.out[static_cast<int64_t>(c) * a.M + r] = o;
    }
  }
}

}  // namespace qmv
