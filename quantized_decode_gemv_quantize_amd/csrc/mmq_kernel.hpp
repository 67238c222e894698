// mmq_kernel.hpp - the many-column path (more activation columns than the
// mat-vec kernels take at their best) for every weight format: int8
// matrix-core (MFMA) products of 16x16 tiles.
//
// Citations: [MMVQ §X] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时
// 一条量化权重如何被 dp4a 逐块点积", section X.
//
// Beyond a handful of columns the per-column integer dots of the mat-vec
// kernels cost more than the weight stream [MMVQ §多个 token 时, §分派]; here
// the weights are decoded once into MFMA operands and reused across 16-column
// tiles, and the integer dots of every (row, column, 32-element block t) come
// from v_mfma_i32_16x16x32_i8: A = 16 rows x 32 codes of block t, B = the
// matching q8_1 block of 16 columns. The block scales are those of the
// mat-vec [MMVQ §一次 vec_dot 的解剖], summed in another order (C_t the int32
// tile of block t, S_t[c] the sum of column c's q8_1 codes in block t, d8_t
// its scale):
//   Q4_K: out += d * sum_t sc_t*C_t*d8_t - dmin * sum_t m_t*(d8_t*S_t)
//         (sc_t*C_t exact below 2^22; the min term, a contraction over the 8
//         sub-blocks, is two fp32 MFMAs per tile and step)
//   Q5_K: as Q4_K with codes 0..31 (bit 4 from qh)
//   Q4_0: out += sum_t d_t*(d8_t*C_t - 8*s_t)      (codes 0..15; s_t the
//         q8_1 block's stored fp16 d8*sum(q), as the mat-vec uses it)
//   Q5_0: out += sum_t d_t*(d8_t*C_t - 16*s_t)     (codes 0..31)
//   Q4_1, Q5_1: out += sum_t d_t*d8_t*C_t + sum_t m_t*s_t (codes 0..15 /
//         0..31; the min term a contraction over the 8 blocks, two fp32
//         MFMAs per tile and step)
//   Q8_0: out += sum_t d_t*d8_t*C_t                (signed codes)
//   Q6_K: out += d * sum_t d8_t*(sc_2t*(C_t,lo - 32*S_t,lo) + sc_2t+1*(C_t,hi - 32*S_t,hi))
//         (codes 0..63; the 16-element sub-blocks 2t and 2t+1 are the two
//         halves of block t, taken by two MFMAs whose B operand keeps only
//         its half; each bracket is an exact integer below 2^23)
//
// A workgroup owns RT x CT tiles (16 rows x 16 columns each); its NW waves
// split the K range (256-weight steps) and their fp32 partials are summed
// through LDS in a fixed order. MFMA lane layouts (checked on the device):
//   i8 A: lane l holds row l%16, codes k = 8*(l/16) .. +7
//   i8 B: lane l holds column l%16, codes k = 8*(l/16) .. +7
//   f32 A: lane l holds row l%16, k = l/16; f32 B: column l%16, k = l/16
//   D (both): lane l holds rows 4*(l/16) .. +3 of column l%16
#pragma once

#include "common.hpp"
#include "formats.hpp"
#include "mmq_plan.hpp"
#include "mmvq_kernel.hpp"     // glu(), the epilogue shared with the row kernels

namespace qmv {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ long pack2(uint32_t lo, uint32_t hi) {
  return static_cast<long>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// LDS accesses of one wave complete in order; the waits make the data
// written by other lanes of the wave visible to the reads that follow.
__device__ __forceinline__ void mmq_lds_fence() {
  __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// 8 bytes at a 2-byte aligned LDS address p, misaligned by MIS (0 or 2)
// bytes from a dword boundary: dword reads re-aligned in registers.
template <int MIS>
__device__ __forceinline__ long lds8(const uint8_t* p) {
  if constexpr (MIS == 0) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
    return pack2(w[0], w[1]);
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p - 2);
    return pack2(__builtin_amdgcn_alignbit(w[1], w[0], 16), __builtin_amdgcn_alignbit(w[2], w[1], 16));
  }
}

// Two dwords at a 2-byte aligned LDS address whose misalignment (0 or 2
// bytes) is known only at run time.
__device__ __forceinline__ u32x2 lds8_rt(const uint8_t* p, int mis) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p - mis);
  const uint32_t w0 = w[0], w1 = w[1], w2 = mis ? w[2] : 0u;
  const uint32_t sh = static_cast<uint32_t>(mis) * 8u;
  u32x2 r;
  r.x = __builtin_amdgcn_alignbit(w1, w0, sh);
  r.y = __builtin_amdgcn_alignbit(w2, w1, sh);
  return r;
}

// The q8_1 block t of the lane's column r16 in the B tile of column tile ct:
// codes 8q..8q+7 (two dword reads: the 36-byte block makes the pair 8-byte
// aligned only in odd blocks) and the block's scale.
template <int CT>
__device__ __forceinline__ long b_operand(const uint8_t (&b)[CT][16][288], int ct, int r16, int q, int t,
                                          float& d8) {
  const uint8_t* blk = &b[ct][r16][36 * t];
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(blk + 4 + 8 * q);
  d8 = h2f(*reinterpret_cast<const uint16_t*>(blk));
  return pack2(cw[0], cw[1]);
}

// Per-row factors of one step, written by the lanes that unpack them and
// read back in the D layout (rows 4q..4q+3 per lane).
template <class F, int RT> struct MmqRowLds;
template <int RT> struct MmqRowLds<Q4K, RT> {
  uint8_t sc[RT][4][16][2];        // sc_t of row, t = 2c + h at [c][row][h]
  float d[RT][16];                 // d of row
};
template <int RT> struct MmqRowLds<Q5K, RT> : MmqRowLds<Q4K, RT> {};
template <int RT> struct MmqRowLds<Q40, RT> { float d[RT][8][16]; };   // d of block t of row
template <int RT> struct MmqRowLds<Q41, RT> { float d[RT][8][16]; };
template <int RT> struct MmqRowLds<Q50, RT> { float d[RT][8][16]; };
template <int RT> struct MmqRowLds<Q51, RT> { float d[RT][8][16]; };
template <int RT> struct MmqRowLds<Q80, RT> { float d[RT][8][16]; };
template <int RT> struct MmqRowLds<Q6K, RT> {
  int8_t sc[RT][16][16];           // scale of sub-block s of row at [s][row]
  float d[RT][16];
};

// One matrix's part of a wave's staging: the step images of its RT x 16
// rows and their per-row factors.
template <class F, int RT>
struct alignas(16) MmqImage {
  uint8_t a[RT][16][MmqGeom<F>::kRowLds];   // the 16 rows' step images
  MmqRowLds<F, RT> x;
};
template <int CT> using MmqBTiles = uint8_t[CT][16][288];   // 16 columns' 8 q8_1 blocks per tile

template <class F, int RT, int CT, int G>
struct MmqWaveLds {
  MmqImage<F, RT> m[G];                      // [0] up (or plain), [1] gate
  MmqBTiles<CT> b;
};

// LDS bytes of a workgroup (the staging tiles of all waves; the reduction
// reuses them), and the shapes that fit one compute unit's 160 KB.
template <class F, int RT, int CT, int NW, int G>
constexpr size_t mmq_lds_bytes() {
  const size_t stage = sizeof(MmqWaveLds<F, RT, CT, G>) * NW, red = sizeof(float) * NW * G * RT * CT * 4 * kWave;
  return stage > red ? stage : red;
}
template <class F, int RT, int CT, int NW, int G>
constexpr bool mmq_fits() { return mmq_lds_bytes<F, RT, CT, NW, G>() <= 160 * 1024; }

// Where the lane's rows sit: tile_off = byte offset of the tile's first row
// from W; row_off(rt) = that of row r16 of row tile rt (clamped to M - 1).
struct MmqRows {
  int64_t tile_off, row_base, M, row_bytes;
  __device__ int64_t row_off(int rt, int r16) const {
    int64_t r = row_base + 16 * rt + r16;
    r = r < M ? r : M - 1;
    return (r - row_base) * row_bytes + tile_off;
  }
};

// One step of a format from the wave's LDS, accumulated into acc[rt][ct][i]
// (row 4q+i of row tile rt, column r16 of column tile ct).
template <class F> struct MmqStep;

// Q4_K and Q5_K (header of Q4_K at step byte 0, the codes of chunk c at
// QS + 32c; Q5_K: qh[32] at byte 16, bit t of qh[l] the fifth bit of element
// l of sub-block t). Lane (r16, q) unpacks sub-blocks 2q and 2q+1 of row
// r16: the f32 A operand of the min term (k = q stands for t = 2q in the
// even product, t = 2q+1 in the odd one) and the scales, which the D layout
// reads back per chunk for rows 4q..4q+3.
template <class F, int QS, bool HB>
struct MmqStepK {
  template <int RT, int CT>
  __device__ static void run(MmqImage<F, RT>& img, const MmqBTiles<CT>& b, const MmqRows&, int, int lane,
                             float (&acc)[RT][CT][4]) {
    const int r16 = lane & 15, q = lane >> 4;
    const Q4K::Lane L = Q4K::lane(2 * q);       // scale unpack of chunk q (sub-blocks 2q, 2q+1)
    const long ones = 0x0101010101010101l;
    float am[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const u32x4 hdr = *reinterpret_cast<const u32x4*>(&img.a[rt][r16][0]);
      uint32_t scp, mp;
      Q4K::chunk_scales(hdr, L, scp, mp);
      *reinterpret_cast<uint16_t*>(&img.x.sc[rt][q][r16][0]) = static_cast<uint16_t>(scp & 0xFFFFu);
      img.x.d[rt][r16] = h2f(hdr.x);
      const float dmin = h2f(hdr.x >> 16);
      am[rt][0] = -dmin * static_cast<float>(mp & 0xFFu);
      am[rt][1] = -dmin * static_cast<float>((mp >> 8) & 0xFFu);
    }
    mmq_lds_fence();

    float accd[RT][CT][4], e[CT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) accd[rt][ct][i] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) e[ct][0] = e[ct][1] = 0.0f;
    // fifth bits of elements 8q..8q+7 (the same bytes for every chunk)
    u32x2 qh[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      qh[rt].x = qh[rt].y = 0u;
      if constexpr (HB) qh[rt] = *reinterpret_cast<const u32x2*>(&img.a[rt][r16][16 + 8 * q]);
    }
    // sub-blocks 2c and 2c+1 share the code bytes of chunk c (low and high
    // nibbles); the chunk loop is kept rolled so only one chunk's operands
    // are live
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      u32x2 w[RT], scw[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        w[rt] = *reinterpret_cast<const u32x2*>(&img.a[rt][r16][QS + 32 * c + 8 * q]);
        scw[rt] = *reinterpret_cast<const u32x2*>(&img.x.sc[rt][c][4 * q][0]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * c + h;
        long A[RT];
        int sc[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          uint32_t lo = (w[rt].x >> (4 * h)) & 0x0F0F0F0Fu, hi = (w[rt].y >> (4 * h)) & 0x0F0F0F0Fu;
          if constexpr (HB) {
            lo |= ((qh[rt].x >> t) & 0x01010101u) << 4;
            hi |= ((qh[rt].y >> t) & 0x01010101u) << 4;
          }
          A[rt] = pack2(lo, hi);
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
          const long B = b_operand<CT>(b, ct, r16, q, t, d8[ct]);
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
      const float4 dv = *reinterpret_cast<const float4*>(&img.x.d[rt][4 * q]);
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
  }
};

template <> struct MmqStep<Q4K> : MmqStepK<Q4K, 16, false> {};
template <> struct MmqStep<Q5K> : MmqStepK<Q5K, 48, true> {};

// The 32-weight block formats: one fp16 scale d per block t (block at byte
// BB*t of the step, its codes CO bytes in). Lane (r16, q) converts the
// scales of blocks 2q and 2q+1 of row r16 for the D layout. Nibble formats:
// byte j of the codes holds element j (low nibble) and j + 16 (high), so
// k-slice q reads bytes 8*(q&1) .. +7 and takes nibble q>>1; with QH >= 0
// the 32-bit word at block byte QH holds the fifth bit of element e at bit
// e, so k-slice q (elements 8q .. 8q+7) takes byte q of it. ZP: the zero
// point as a multiple of the q8_1 block's stored s (its fp16 d8*sum(q)), as
// in the mat-vec: Q4_0 -8, Q5_0 -16. MIN: Q4_1 / Q5_1, the fp16 min m at
// block byte 2 times s, summed over the 8 blocks of the step by two fp32
// MFMAs per tile (lane (r16, q) supplies m of blocks 2q + h of row r16 and s
// of blocks 2q + h of column r16). Q8_0: k-slice q reads code bytes
// 8q .. 8q+7 as they are.
template <class F, int BB, int CO, bool NIBBLES, int QH, int ZP, bool MIN>
struct MmqStepBlocks {
  template <int RT, int CT>
  __device__ static void run(MmqImage<F, RT>& img, const MmqBTiles<CT>& b, const MmqRows&, int, int lane, float (&acc)[RT][CT][4]) {
    const int r16 = lane & 15, q = lane >> 4;
    float am[RT][2], e[CT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * q + h;
        img.x.d[rt][t][r16] = h2f(*reinterpret_cast<const uint16_t*>(&img.a[rt][r16][BB * t]));
        am[rt][h] = MIN ? h2f(*reinterpret_cast<const uint16_t*>(&img.a[rt][r16][BB * t + 2])) : 0.0f;
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        e[ct][h] = MIN ? h2f(*reinterpret_cast<const uint16_t*>(&b[ct][r16][36 * (2 * q + h) + 2])) : 0.0f;
    mmq_lds_fence();
    const int nib = 4 * (q >> 1);
    static_for<0, 8>([&](auto tc) QMV_INLINE {
      constexpr int t = decltype(tc)::value;
      // code bytes of this lane in block t: 2-byte aligned, misaligned by a
      // compile-time 0 or 2 bytes from a dword (BB and CO even; 8*(q&1) and
      // 8q are multiples of 4)
      constexpr int kMis = (BB * t + CO) % 4;
      long A[RT];
      float dw[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint8_t* p = &img.a[rt][r16][BB * t + CO + (NIBBLES ? 8 * (q & 1) : 8 * q)];
        const long raw = lds8<kMis>(p);
        if constexpr (NIBBLES) {
          uint32_t lo = static_cast<uint32_t>(raw), hi = static_cast<uint32_t>(static_cast<uint64_t>(raw) >> 32);
          lo = (lo >> nib) & 0x0F0F0F0Fu;
          hi = (hi >> nib) & 0x0F0F0F0Fu;
          if constexpr (QH >= 0) {
            // bit i of the byte goes to bit 4 of byte i (4 bits per word:
            // the multiply places bit i at bit 8i, the partial products do
            // not overlap)
            const uint32_t hb = img.a[rt][r16][BB * t + QH + q];
            lo |= (((hb & 0xFu) * 0x00204081u) & 0x01010101u) << 4;
            hi |= (((hb >> 4) * 0x00204081u) & 0x01010101u) << 4;
          }
          A[rt] = pack2(lo, hi);
        } else {
          A[rt] = raw;
        }
        const float4 dv = *reinterpret_cast<const float4*>(&img.x.d[rt][t][4 * q]);
        dw[rt][0] = dv.x; dw[rt][1] = dv.y; dw[rt][2] = dv.z; dw[rt][3] = dv.w;
      }
      v4i C[RT][CT];
      float d8[CT], zs[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const long B = b_operand<CT>(b, ct, r16, q, t, d8[ct]);
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) C[rt][ct] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], B, zero, 0, 0, 0);
        zs[ct] = 0.0f;
        if constexpr (ZP != 0)
          zs[ct] = static_cast<float>(ZP) * h2f(*reinterpret_cast<const uint16_t*>(&b[ct][r16][36 * t + 2]));
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[rt][ct][i] = fmaf(fmaf(static_cast<float>(C[rt][ct][i]), d8[ct], zs[ct]), dw[rt][i], acc[rt][ct][i]);
    });
    if constexpr (MIN) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          v4f v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[rt][ct][i];
          v = __builtin_amdgcn_mfma_f32_16x16x4f32(am[rt][0], e[ct][0], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x4f32(am[rt][1], e[ct][1], v, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rt][ct][i] = v[i];
        }
    }
  }
};
//                                                   BB  CO  NIB    QH  ZP   MIN
template <> struct MmqStep<Q40> : MmqStepBlocks<Q40, 18, 2, true, -1, -8, false> {};
template <> struct MmqStep<Q41> : MmqStepBlocks<Q41, 20, 4, true, -1, 0, true> {};
template <> struct MmqStep<Q50> : MmqStepBlocks<Q50, 22, 6, true, 2, -16, false> {};
template <> struct MmqStep<Q51> : MmqStepBlocks<Q51, 24, 8, true, 4, 0, true> {};
template <> struct MmqStep<Q80> : MmqStepBlocks<Q80, 34, 2, false, -1, 0, false> {};

// Q6_K super-block at image byte base = 16 - delta of each row (delta per
// row and step): ql[128] @0, qh[64] @128, int8 sc[16] @192, fp16 d @208.
// Element e = 128h + 32g + l of block t = 4h + g: low 4 bits in ql[64h +
// 32(g%2) + l] (nibble g/2), high 2 bits at bit 2g of qh[32h + l]. Lane
// (r16, q) copies the scales of sub-blocks 4q..4q+3 of row r16 (and q = 0
// its d) for the D layout.
template <> struct MmqStep<Q6K> {
  template <int RT, int CT>
  __device__ static void run(MmqImage<Q6K, RT>& im, const MmqBTiles<CT>& b, const MmqRows& rows, int sb, int lane,
                             float (&acc)[RT][CT][4]) {
    const int r16 = lane & 15, q = lane >> 4;
    int base[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      base[rt] = MmqGeom<Q6K>::image_base(rows.row_off(rt, r16), sb);
      const uint8_t* img = &im.a[rt][r16][base[rt]];
      const u32x2 s4 = lds8_rt(img + 192 + 4 * q, base[rt] & 2);   // scales 4q..4q+3 (and 4 more)
#pragma unroll
      for (int k = 0; k < 4; ++k) im.x.sc[rt][4 * q + k][r16] = static_cast<int8_t>((s4.x >> (8 * k)) & 0xFFu);
      if (q == 0) im.x.d[rt][r16] = h2f(*reinterpret_cast<const uint16_t*>(img + 208));
    }
    mmq_lds_fence();
    const long ones = 0x0101010101010101l;
    float accd[RT][CT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) accd[rt][ct][i] = 0.0f;
#pragma unroll 2
    for (int t = 0; t < 8; ++t) {
      const int h = t >> 2, g = t & 3;
      long A[RT];
      int sc[RT][2][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint8_t* img = &im.a[rt][r16][base[rt]];
        const int mis = base[rt] & 2;
        const u32x2 ql = lds8_rt(img + 64 * h + 32 * (g & 1) + 8 * q, mis);
        const u32x2 qh = lds8_rt(img + 128 + 32 * h + 8 * q, mis);
        const int ns = 4 * (g >> 1), hs = 2 * g;
        A[rt] = pack2(((ql.x >> ns) & 0x0F0F0F0Fu) | (((qh.x >> hs) & 0x03030303u) << 4),
                      ((ql.y >> ns) & 0x0F0F0F0Fu) | (((qh.y >> hs) & 0x03030303u) << 4));
        const uint32_t s0 = *reinterpret_cast<const uint32_t*>(&im.x.sc[rt][2 * t][4 * q]);
        const uint32_t s1 = *reinterpret_cast<const uint32_t*>(&im.x.sc[rt][2 * t + 1][4 * q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[rt][0][i] = sbfe(s0, 8 * i, 8);
          sc[rt][1][i] = sbfe(s1, 8 * i, 8);
        }
      }
      // the sub-block halves of block t: k-slices 0, 1 (lanes q < 2) and 2, 3
      const bool lo_half = q < 2;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float d8;
        const long B = b_operand<CT>(b, ct, r16, q, t, d8);
        const long Blo = lo_half ? B : 0l, Bhi = lo_half ? 0l : B;
        const v4i zero = {0, 0, 0, 0};
        const int S32lo = 32 * __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, Blo, zero, 0, 0, 0)[0];
        const int S32hi = 32 * __builtin_amdgcn_mfma_i32_16x16x32_i8(ones, Bhi, zero, 0, 0, 0)[0];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const v4i Clo = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], Blo, zero, 0, 0, 0);
          const v4i Chi = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt], Bhi, zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = mul24(sc[rt][0][i], Clo[i] - S32lo) + mul24(sc[rt][1][i], Chi[i] - S32hi);
            accd[rt][ct][i] = fmaf(static_cast<float>(v), d8, accd[rt][ct][i]);
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float4 dv = *reinterpret_cast<const float4*>(&im.x.d[rt][4 * q]);
      const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rt][ct][i] = fmaf(dd[i], accd[rt][ct][i], acc[rt][ct][i]);
    }
  }
};

// Largest magnitude of the 32 fp32 values of a staged block: each v_max3
// takes two magnitudes (the values are finite, so the NaN quieting that a
// plain fmaxf adds per operand is not needed); equal to the quantizer's
// amax, since a maximum is exact in any order.
__device__ __forceinline__ float block_amax(const u32x4 (&v)[8]) {
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    asm("v_max3_f32 %0, |%1|, |%2|, %0" : "+v"(m0) : "v"(v[k].x), "v"(v[k].y));
    asm("v_max3_f32 %0, |%1|, |%2|, %0" : "+v"(m1) : "v"(v[k].z), "v"(v[k].w));
  }
  return fmaxf(m0, m1);
}

// G = 2: the gate/up form. The up (W) and gate (Wg) rows of a tile are
// staged side by side and each runs the format's step against the same B
// tiles; the epilogue sums both over the waves and applies the scales,
// biases and GLU of the row kernels' epilogue.
//
// XF: the columns arrive as fp32 (the fused form). Each lane quantizes the
// q8_1 blocks it staged, with the stand-alone quantizer's arithmetic (same
// amax, scale, codes and fp16 {d, s}), and writes them into the B tiles, so
// the tiles and the result are those of the q8_1 form bit for bit.
template <class F, int RT, int CT, int NW, int G, bool XF>
__global__ void __launch_bounds__(NW * kWave, 8 / NW) mmq_kernel(MmqArgs a) {
  using Gm = MmqGeom<F>;
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int r16 = lane & 15, q = lane >> 4;
  int64_t bx;
  int by;
  mmq_tile_of(blockIdx.x, a.gx, a.gy, bx, by);
  const int64_t row_base = bx * (16 * RT);
  const int col_base = by * (16 * CT);
  const int sb0 = mmq_sb_begin(a.nsb, wave, NW), sb1 = mmq_sb_begin(a.nsb, wave + 1, NW);
  const MmqRows rows{row_base * a.row_bytes, row_base, a.M, a.row_bytes};

  // the staging tiles of the NW waves; after the K loop the same LDS holds
  // the partial sums of the reduction
  constexpr int NV = RT * CT * 4;
  __shared__ __align__(16) uint8_t smem[mmq_lds_bytes<F, RT, CT, NW, G>()];
  MmqWaveLds<F, RT, CT, G>& lds = reinterpret_cast<MmqWaveLds<F, RT, CT, G>*>(smem)[wave];
  float acc[G][RT][CT][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][rt][ct][i] = 0.0f;

  MmqOffsets<F, RT, CT> off;
  // staged loads -> LDS: A loads into their rows' images, B piece k at byte
  // 16k of the B tiles (fp32 columns: each staged block quantized into its
  // 36 bytes at column * 288 + block * 36)
  auto store_a = [&](const MmqStage<F, RT, CT, G, XF>& st, int sb) QMV_INLINE {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint8_t* la = &lds.m[g].a[0][0][0];
#pragma unroll
      for (int j = 0; j < mmq_a_slots<F, RT>(); ++j) {
        if (lane + kWave * j < mmq_a_pieces<F>() * RT) {
          uint8_t* dst = la + off.arow[j] * Gm::kRowLds + Gm::piece_lds(rows.tile_off + off.a[j], sb, off.apc[j]);
          if (Gm::piece_short(off.apc[j])) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(st.a[g][j].x);
          else *reinterpret_cast<u32x4*>(dst) = st.a[g][j];
        }
      }
    }
  };
  // (fp32 columns: each slot's registers take the next step's values as
  // soon as the slot is quantized)
  auto store_b = [&](MmqStage<F, RT, CT, G, XF>& st, int next) QMV_INLINE {
    uint8_t* lb = &lds.b[0][0][0];
    if constexpr (XF) {
#pragma unroll
      for (int j = 0; j < mmq_x_slots<CT>(); ++j) {
        int col, blk, c;
        mmq_x_pair(lane, j, 0, a.n, col, blk, c);
        const float d = q8_scale(block_amax(st.x[j]));
        uint32_t codes[8];
        int sq = 0;
        q8_quant_block<8>(st.x[j], d, codes, sq);
        mmq_stage_load_x<F, RT, CT, G>(a, col_base, lane, next, j, st);
        uint32_t* dst = reinterpret_cast<uint32_t*>(lb + col * 288 + blk * 36);
        dst[0] = f2h_bits(d) | (f2h_bits(q8_s(d, sq)) << 16);
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[1 + k] = codes[k];
      }
    } else {
#pragma unroll
      for (int j = 0; j < mmq_b_slots<CT>(); ++j) {
        const int k = lane + kWave * j;
        if (k < kMmqBPieces * CT) *reinterpret_cast<u32x4*>(lb + 16 * k) = st.b[j];
      }
    }
  };

  // Pipeline: the staging loads of step sb+1 are in flight while sb is
  // computed from LDS. The prefetch is unconditional (past the end it
  // re-reads the last step, from cache) so every path has the same loads in
  // flight. (Two steps in flight, in a second register buffer, measured
  // slower at 16 columns: 16.3 -> 17.3 us at 4096x14336.) The fp32 form
  // issues the next weights before it quantizes the staged columns, and the
  // next values of each column slot once that slot is quantized.
  if (sb0 < sb1) {
    mmq_offsets<F, RT, CT>(a, row_base, col_base, lane, off);
    MmqStage<F, RT, CT, G, XF> st;
    mmq_stage_load<F, RT, CT, G, XF>(a, row_base, col_base, lane, sb0, off, st);
    for (int sb = sb0; sb < sb1; ++sb) {
      mmq_lds_fence();             // the previous step's reads are done
      const int next = sb + 1 < sb1 ? sb + 1 : sb;
      store_a(st, sb);
      if constexpr (XF) {
        mmq_stage_load_a<F, RT, CT, G, XF>(a, row_base, lane, next, off, st);
        __builtin_amdgcn_sched_barrier(0);
        store_b(st, next);
      } else {
        store_b(st, next);
        mmq_stage_load<F, RT, CT, G, XF>(a, row_base, col_base, lane, next, off, st);
      }
      __builtin_amdgcn_sched_barrier(0);
      mmq_lds_fence();
#pragma unroll
      for (int g = 0; g < G; ++g) MmqStep<F>::template run<RT, CT>(lds.m[g], lds.b, rows, sb, lane, acc[g]);
    }
  }

  // ---- sum the waves' partials (in wave order), epilogue, store
  __syncthreads();                 // every wave is done with its staging tiles
  float(*red)[G][NV][kWave] = reinterpret_cast<float(*)[G][NV][kWave]>(smem);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][g][(rt * CT + ct) * 4 + i][lane] = acc[g][rt][ct][i];
  __syncthreads();
  for (int v = wave; v < NV; v += NW) {
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s[g] = red[0][g][v][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s[g] += red[w][g][v][lane];
    }
    int64_t r;
    int c;
    mmq_store_pos<RT, CT>(v, q, r16, row_base, col_base, r, c);
    if (r < a.M && c < a.n) {
      float up = s[0];
      if (a.up_scale) up *= a.up_scale[0];
      if (a.up_bias) up += a.up_bias[r];
      float o = up;
      if constexpr (G == 2) {
        float gate = s[G - 1];
        if (a.gate_scale) gate *= a.gate_scale[0];
        if (a.gate_bias) gate += a.gate_bias[r];
        o = glu(a.glu_op, gate, up, a.glu_limit);
      }
      a.out[static_cast<int64_t>(c) * a.M + r] = o;
    }
  }
}

}  // namespace qmv
