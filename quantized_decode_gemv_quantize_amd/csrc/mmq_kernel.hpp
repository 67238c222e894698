// mmq_kernel.hpp - the many-column path (n > 8 activation columns) for
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
// matching q8_1 block of 16 columns. The block scales are applied to each
// sub-block's int32 tile afterwards, as in the mat-vec [MMVQ §一次 vec_dot 的解剖]:
//   out[r][c] += d*sc_t[r] * d8_t[c] * C_t[r][c] - dmin*m_t[r] * d8_t[c] * S_t[c]
// with S_t[c] = sum of the q8_1 codes of column c in block t, itself an MFMA
// of an all-ones A with the same B.
//
// A workgroup owns RT x CT tiles (16 rows x 16 columns each); its NW waves
// split the K range (super-blocks) and their fp32 partials are summed through
// LDS in a fixed order. MFMA lane layouts (checked on the device):
//   A: lane l holds row l%16, codes k = 8*(l/16) .. +7
//   B: lane l holds column l%16, codes k = 8*(l/16) .. +7
//   D: lane l holds rows 4*(l/16) .. +3 of column l%16
#pragma once

#include "common.hpp"
#include "formats.hpp"
#include "mmq_plan.hpp"

namespace qmv {

typedef int v4i __attribute__((ext_vector_type(4)));


__device__ __forceinline__ long pack2(uint32_t lo, uint32_t hi) {
  return static_cast<long>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// LDS of one wave: the staged super-block tiles and the row factors.
template <int RT, int CT>
struct MmqWaveLds {
  uint8_t a[RT][16][144];          // 16 rows' super-blocks
  uint8_t b[CT][16][288];          // 16 columns' 8 q8_1 blocks
  float fac[RT][2][8][16];         // d*sc, dmin*m of sub-block t, row
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
__global__ void __launch_bounds__(NW * kWave) mmq_q4k_kernel(MmqArgs a) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (16 * RT);
  const int col_base = static_cast<int>(blockIdx.y) * (16 * CT);
  const int sb0 = mmq_sb_begin(a.nsb, wave, NW), sb1 = mmq_sb_begin(a.nsb, wave + 1, NW);
  const Q4K::Lane L = Q4K::lane(2 * q);       // scale unpack of chunk q (sub-blocks 2q, 2q+1)
  const long ones = 0x0101010101010101l;

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

  // staged pieces -> LDS (the same lane-to-piece map as the loads)
  auto store_stage = [&](const MmqStage<RT, CT>& st) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < kMmqAPerLane; ++j) {
        const int k = lane + kWave * j;
        if (k < kMmqAPieces) *reinterpret_cast<u32x4*>(&lds.a[rt][k / 9][16 * (k % 9)]) = st.a[rt][j];
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int j = 0; j < kMmqBPerLane; ++j) {
        const int k = lane + kWave * j;
        if (k < kMmqBPieces) *reinterpret_cast<u32x4*>(&lds.b[ct][k / 18][16 * (k % 18)]) = st.b[ct][j];
      }
  };

  // LDS accesses of one wave complete in order; the waits make the data
  // written by other lanes of the wave visible to the reads that follow
  auto lds_fence = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };

  // one super-block from LDS: row factors, then 8 sub-blocks of MFMAs, each
  // int32 tile scaled into the fp32 accumulators
  auto compute = [&]() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const u32x4 hdr = *reinterpret_cast<const u32x4*>(&lds.a[rt][r16][0]);
      uint32_t scp, mp;
      Q4K::chunk_scales(hdr, L, scp, mp);
      const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
      lds.fac[rt][0][2 * q][r16] = d * static_cast<float>(scp & 0xFFu);
      lds.fac[rt][0][2 * q + 1][r16] = d * static_cast<float>((scp >> 8) & 0xFFu);
      lds.fac[rt][1][2 * q][r16] = dmin * static_cast<float>(mp & 0xFFu);
      lds.fac[rt][1][2 * q + 1][r16] = dmin * static_cast<float>((mp >> 8) & 0xFFu);
    }
    lds_fence();
    // sub-blocks 2c and 2c+1 share the code bytes of chunk c (low and high
    // nibbles); the chunk loop is kept rolled so only one chunk's operands
    // are live
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      u32x2 w[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) w[rt] = *reinterpret_cast<const u32x2*>(&lds.a[rt][r16][16 + 32 * c + 8 * q]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * c + h;
        long A[RT];
        float4 fd[RT], fm[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          A[rt] = pack2((w[rt].x >> (4 * h)) & 0x0F0F0F0Fu, (w[rt].y >> (4 * h)) & 0x0F0F0F0Fu);
          fd[rt] = *reinterpret_cast<const float4*>(&lds.fac[rt][0][t][4 * q]);
          fm[rt] = *reinterpret_cast<const float4*>(&lds.fac[rt][1][t][4 * q]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const uint8_t* blk = &lds.b[ct][r16][36 * t];
          const u32x2 cw = *reinterpret_cast<const u32x2*>(blk + 4 + 8 * q);
          const long B = pack2(cw.x, cw.y);
          const float d8 = h2f(*reinterpret_cast<const uint16_t*>(blk));
          const v4i zero = {0, 0, 0, 0};
          const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, B, zero, 0, 0, 0);
          const float d8s = d8 * static_cast<float>(S[0]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const v4i C = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], B, zero, 0, 0, 0);
            const float f[4] = {fd[rt].x, fd[rt].y, fd[rt].z, fd[rt].w};
            const float m[4] = {fm[rt].x, fm[rt].y, fm[rt].z, fm[rt].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[rt][ct][i] = fmaf(static_cast<float>(C[i]), f[i] * d8, fmaf(-m[i], d8s, acc[rt][ct][i]));
          }
        }
      }
    }
  };

  // Pipeline: the staging loads of super-block sb+1 are in flight while sb
  // is computed from LDS. The prefetch is unconditional (past the end it
  // re-reads the last super-block, from cache) so every path has the same
  // loads in flight.
  if (sb0 < sb1) {
    MmqStage<RT, CT> st;
    mmq_stage_load<RT, CT>(a, row_base, col_base, lane, sb0, st);
    for (int sb = sb0; sb < sb1; ++sb) {
      lds_fence();                 // the previous super-block's reads are done
      store_stage(st);
      const int next = sb + 1 < sb1 ? sb + 1 : sb;
      mmq_stage_load<RT, CT>(a, row_base, col_base, lane, next, st);
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
