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
// A workgroup owns RT x CT tiles (16 rows x 16 columns each); its four waves
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

template <int RT, int CT>
__global__ void __launch_bounds__(kMmqWaves * kWave) mmq_q4k_kernel(MmqArgs a) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (16 * RT);
  const int col_base = static_cast<int>(blockIdx.y) * (16 * CT);
  const int sb0 = mmq_sb_begin(a.nsb, wave), sb1 = mmq_sb_begin(a.nsb, wave + 1);
  const uint8_t* arow[RT];
  const uint8_t* bcol[CT];
  bool bvalid[CT];
  mmq_pointers<RT, CT>(a, row_base, col_base, r16, arow, bcol, bvalid);
  const Q4K::Lane L = Q4K::lane(2 * q);       // scale unpack of chunk q (sub-blocks 2q, 2q+1)
  const long ones = 0x0101010101010101l;

  // per wave: d*sc and dmin*m of sub-block t of the tile's 16 rows
  __shared__ __align__(16) float fac[kMmqWaves][RT][2][8][16];
  float acc[RT][CT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][ct][i] = 0.0f;

  for (int sb = sb0; sb < sb1; ++sb) {
    // ---- loads: codes of chunk q of each row, the rows' headers, the q8_1
    // codes and scales of the 8 blocks of every column
    MmqQ4KLoads<RT, CT> ld;
    mmq_q4k_load(arow, bcol, sb, q, ld);
    const u32x4 (&hdr)[RT] = ld.hdr;
    const u32x2 (&qs)[RT][4] = ld.qs;
    const u32x2 (&yq)[CT][8] = ld.yq;
    const uint32_t (&yd)[CT][8] = ld.yd;

    // ---- row factors of this lane's row, sub-blocks 2q and 2q+1 -> LDS
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t scp, mp;
      Q4K::chunk_scales(hdr[rt], L, scp, mp);
      const float d = h2f(hdr[rt].x), dmin = h2f(hdr[rt].x >> 16);
      fac[wave][rt][0][2 * q][r16] = d * static_cast<float>(scp & 0xFFu);
      fac[wave][rt][0][2 * q + 1][r16] = d * static_cast<float>((scp >> 8) & 0xFFu);
      fac[wave][rt][1][2 * q][r16] = dmin * static_cast<float>(mp & 0xFFu);
      fac[wave][rt][1][2 * q + 1][r16] = dmin * static_cast<float>((mp >> 8) & 0xFFu);
    }
    // the same wave reads them back in the result layout: LDS operations of
    // one wave complete in order; wait for the writes before the reads
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = t >> 1, sh = 4 * (t & 1);
      long A[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        A[rt] = pack2((qs[rt][c].x >> sh) & 0x0F0F0F0Fu, (qs[rt][c].y >> sh) & 0x0F0F0F0Fu);
      float fd[RT][4], fm[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fd[rt][i] = fac[wave][rt][0][t][4 * q + i];
          fm[rt][i] = fac[wave][rt][1][t][4 * q + i];
        }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const long B = bvalid[ct] ? pack2(yq[ct][t].x, yq[ct][t].y) : 0l;
        const v4i zero = {0, 0, 0, 0};
        const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, B, zero, 0, 0, 0);
        const float d8 = bvalid[ct] ? h2f(yd[ct][t]) : 0.0f;
        const float d8s = d8 * static_cast<float>(S[0]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const v4i C = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], B, zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[rt][ct][i] = fmaf(static_cast<float>(C[i]), fd[rt][i] * d8, fmaf(-fm[rt][i], d8s, acc[rt][ct][i]));
        }
      }
    }
    // the next super-block rewrites fac: this wave's reads come first (in order)
    __builtin_amdgcn_wave_barrier();
  }

  // ---- sum the four waves' partials (fixed order) and store
  constexpr int NV = RT * CT * 4;
  __shared__ float red[kMmqWaves][NV][kWave];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(rt * CT + ct) * 4 + i][lane] = acc[rt][ct][i];
  __syncthreads();
  for (int v = wave; v < NV; v += kMmqWaves) {
    const float s = ((red[0][v][lane] + red[1][v][lane]) + red[2][v][lane]) + red[3][v][lane];
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
