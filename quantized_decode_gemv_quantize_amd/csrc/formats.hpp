// formats.hpp - GGUF-style weight blocks and the q8_1 activation block, as
// seen by one lane of the MMVQ kernels.
//
// Citations: [MMVQ §X] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时
// 一条量化权重如何被 dp4a 逐块点积", section X; [GGUF16 §X] = page "GGUF 量化内幕：
// 第16章 llama.cpp 量化代码架构", section X.
//
// Work unit. A row of K weights is cut into units, one per lane of the team
// that owns the row; a lane keeps the same unit for every row it processes,
// so it loads the matching activation codes once and keeps them in
// registers. Units are chosen so that a wave's weight loads for one row are
// contiguous 16-byte pieces:
//   Q4_K: unit = 16 bytes of codes of one super-block (32 weights; 8 units
//         per super-block), plus that super-block's 16-byte header.
//   Q4_0: unit = one 18-byte block (32 weights).
//   Q6_K: unit = one quarter of a super-block (64 weights): 2 x 16 bytes of
//         low bits, 16 bytes of high bits, 4 int8 scales, the fp16 d.
//
// Each format provides:
//   Act           activation registers of one column for the lane's unit
//   issue_act     issue the loads of the lane's slice of a q8_1 column into
//                 Act (codes in place, fp16 scale bits held as raw words)
//   finish_act    turn the raw scale bits into the fp32 values col_dot uses
//                 (split from issue_act so the weight loads can be issued
//                 before anything waits for the activation)
//   load_act      issue_act then finish_act
//   load_x        load the lane's fp32 activation values (XRaw, kXWords
//                 words) of one column
//   quant_x       quantize them to the Act of load_act, with the q8_1
//                 quantizer's own arithmetic (same codes and scales as
//                 load_act after mmvq_quantize_q8_1); lanes u and u ^ 1
//                 exchange block maxima, so every lane of the wave runs it
//   Wt            raw weight words of the lane's unit in one row
//   load_wt       issue the loads of Wt
//   Dec / decode  per-row decode shared by all columns (codes, scales)
//   col_dot       the unit's fp32 contribution for one column
//   int_dots      the unit's integer dots, added into the block's dot array
//                 (test support: the same decode, no scaling)
#pragma once

#include "common.hpp"
#include "q8.hpp"

namespace qmv {

constexpr int kQ8Bytes = 36;     // fp16 d, fp16 s, 32 x int8   [MMVQ §激活的量化]

// Sum of the 4 signed bytes of a word, via a dot with 0x01010101 (the pages'
// trick for the activation sum of a sub-block [MMVQ §一次 vec_dot 的解剖]).
__device__ __forceinline__ int bsum4(uint32_t w, int c) { return dot4(w, 0x01010101u, c); }

// ===========================================================================
// Q4_K  [GGUF16 §16.1.2, §16.2.1; MMVQ §权重的排法, §一次 vec_dot 的解剖]
// 144 bytes: fp16 d @0, fp16 dmin @2, 12 bytes of packed 6-bit scales and
// mins @4, 128 bytes of nibbles @16. Sub-block t (32 weights) of 64-element
// chunk c = t/2 reads the low (t even) or high (t odd) nibbles of
// qs[32c .. 32c+31]. Weight = d*sc_t*q - dmin*m_t.
// Unit u: super-block sb = u/8, p = u%8, chunk c = p/2, half = p%2: the 16
// code bytes qs[32c + 16*half ..] hold elements 16*half .. 16*half+15 of
// sub-blocks t0 = 2c (low nibbles) and t1 = 2c+1 (high nibbles). A wave's 64
// lanes read 8 super-blocks' codes as 8 contiguous 128-byte runs.
// ===========================================================================
struct Q4K {
  static constexpr int kType = 12, kQK = 256, kBlockBytes = 144;
  static constexpr int kUnitsPerBlock = 8, kDotsPerBlock = 16;

  struct Act {
    uint32_t y0[4], y1[4];   // activation codes paired with the t0 / t1 nibbles
    float d0, d1;            // q8_1 scales of the two sub-blocks
    float s0, s1;            // d8 * (sum of the 16 codes): exact in fp32
  };

  __device__ static void act_codes(const uint8_t* ycol, int u, uint32_t (&q0)[4], uint32_t (&q1)[4],
                                   const uint8_t*& b0, const uint8_t*& b1) {
    const int sb = u >> 3, p = u & 7, c = p >> 1, half = p & 1;
    b0 = ycol + static_cast<int64_t>(8 * sb + 2 * c) * kQ8Bytes;
    b1 = b0 + kQ8Bytes;
    const u32x4 a0 = ld_x4(b0 + 4 + 16 * half), a1 = ld_x4(b1 + 4 + 16 * half);
    q0[0] = a0.x; q0[1] = a0.y; q0[2] = a0.z; q0[3] = a0.w;
    q1[0] = a1.x; q1[1] = a1.y; q1[2] = a1.z; q1[3] = a1.w;
  }

  __device__ static int sum4(const uint32_t (&q)[4]) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) s = bsum4(q[k], s);
    return s;
  }

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const uint8_t *b0, *b1;
    act_codes(ycol, u, a.y0, a.y1, b0, b1);
    a.d0 = __uint_as_float(ld_u16(b0));
    a.d1 = __uint_as_float(ld_u16(b1));
  }

  __device__ static void finish_act(Act& a) {
    a.d0 = h2f(__float_as_uint(a.d0));
    a.d1 = h2f(__float_as_uint(a.d1));
    a.s0 = a.d0 * static_cast<float>(sum4(a.y0));
    a.s1 = a.d1 * static_cast<float>(sum4(a.y1));
  }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  // fp32 activations: the lane holds half of each of its two q8_1 blocks
  // (16 values each); the lane next to it (unit u ^ 1) holds the other
  // halves, so one exchange gives each block's amax.
  struct XRaw {
    u32x4 r0[4], r1[4];
  };
  static constexpr int kXWords = 32;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const int sb = u >> 3, p = u & 7, c = p >> 1, half = p & 1;
    const float* x0 = xcol + static_cast<int64_t>(8 * sb + 2 * c) * 32 + 16 * half;
    const float* x1 = x0 + 32;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x.r0[k] = ld_x4(reinterpret_cast<const uint8_t*>(x0 + 4 * k));
      x.r1[k] = ld_x4(reinterpret_cast<const uint8_t*>(x1 + 4 * k));
    }
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
    float m0 = absmax4(x.r0[0]), m1 = absmax4(x.r1[0]);
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      m0 = fmaxf(m0, absmax4(x.r0[k]));
      m1 = fmaxf(m1, absmax4(x.r1[k]));
    }
    const float d0 = q8_scale(max_with_pair(m0)), d1 = q8_scale(max_with_pair(m1));
    int s0 = 0, s1 = 0;
    q8_quant_block(x.r0, d0, a.y0, s0);
    q8_quant_block(x.r1, d1, a.y1, s1);
    a.d0 = q8_d_rounded(d0);
    a.d1 = q8_d_rounded(d1);
    a.s0 = a.d0 * static_cast<float>(s0);
    a.s1 = a.d1 * static_cast<float>(s1);
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { a.y0[k] = 0; a.y1[k] = 0; }
    a.d0 = a.d1 = a.s0 = a.s1 = 0.0f;
  }

  // Per-lane constants, computed once: byte offsets inside a row, and the
  // shifts and masks that pick this lane's two 6-bit scales and mins out of
  // the 12 packed bytes. With scale words H1 = bytes 0..3, H2 = 4..7,
  // H3 = 8..11 and sh = 16*(c%2), sub-blocks 2c, 2c+1 take
  //   c < 2 : sc = (H1 >> sh) & 0x3F3F,   m = (H2 >> sh) & 0x3F3F
  //   c >= 2: sc = ((H3 >> sh) & 0x0F0F)     | ((H1 >> (sh+2)) & 0x3030),
  //           m  = ((H3 >> (sh+4)) & 0x0F0F) | ((H2 >> (sh+2)) & 0x3030)
  // (one byte per sub-block): the pages' branch-free unpack with the scale
  // words read as little-endian 16-bit words.
  struct Lane {
    uint32_t qoff, hoff;       // code bytes and header, from the row start
    uint32_t sh, shm, maskA, maskB;
    bool lo;                   // c < 2
  };
  __device__ static Lane lane(int u) {
    Lane l;
    const int sb = u >> 3, p = u & 7, c = p >> 1;
    l.hoff = static_cast<uint32_t>(sb * kBlockBytes);
    l.qoff = l.hoff + 16 + 16 * p;
    l.lo = c < 2;
    l.sh = 16u * (c & 1);
    l.shm = l.lo ? l.sh : l.sh + 4;
    l.maskA = l.lo ? 0x3F3Fu : 0x0F0Fu;
    l.maskB = l.lo ? 0u : 0x3030u;
    return l;
  }

  struct Wt {
    u32x4 qs;    // 16 code bytes
    u32x4 hdr;   // d | dmin, scales[0..3], scales[4..7], scales[8..11]
  };

  // row: wave-uniform row start (16-byte aligned: 144-byte blocks, 16-byte
  // base); extra: per-lane byte offset added to it
  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    w.hdr = ld_x4(row + (extra + l.hoff));
    w.qs = ld_a16_x4(row + (extra + l.qoff));
  }

  struct Dec {
    uint32_t lo[4], hi[4];   // nibbles of t0 and t1 as unsigned bytes
    uint32_t scp;            // sc of t0 (byte 0) and t1 (byte 1)
    float m0, m1, d, dmin;
  };

  __device__ static void decode(const Wt& w, Dec& o, const Lane& l) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.lo[k] = w.qs[k] & 0x0F0F0F0Fu;
      o.hi[k] = (w.qs[k] >> 4) & 0x0F0F0F0Fu;
    }
    o.d = h2f(w.hdr.x);
    o.dmin = h2f(w.hdr.x >> 16);
    uint32_t mp;
    chunk_scales(w.hdr, l, o.scp, mp);
    o.m0 = static_cast<float>(mp & 0xFFu);
    o.m1 = static_cast<float>((mp >> 8) & 0xFFu);
  }

  // The 6-bit scales (scp) and mins (mp) of the lane's chunk c: byte 0 for
  // sub-block 2c, byte 1 for 2c+1 (the unpack rule above).
  __device__ static void chunk_scales(const u32x4& hdr, const Lane& l, uint32_t& scp, uint32_t& mp) {
    const uint32_t H1 = hdr.y, H2 = hdr.z, H3 = hdr.w;
    const uint32_t Xs = l.lo ? H1 : H3, Xm = l.lo ? H2 : H3;
    scp = ((Xs >> l.sh) & l.maskA) | ((H1 >> (l.sh + 2)) & l.maskB);
    mp = ((Xm >> l.shm) & l.maskA) | ((H2 >> (l.sh + 2)) & l.maskB);
  }

  __device__ static void nibble_dots(const Dec& o, const Act& a, int& dot0, int& dot1) {
    dot0 = 0;
    dot1 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      dot0 = dot4(o.lo[k], a.y0[k], dot0);
      dot1 = dot4(o.hi[k], a.y1[k], dot1);
    }
  }

  // d * (sc0*d8_0*dot0 + sc1*d8_1*dot1) - dmin * (m0*d8_0*S0 + m1*d8_1*S1)
  __device__ static float col_dot(const Dec& o, const Act& a) {
    int dot0, dot1;
    nibble_dots(o, a, dot0, dot1);
    const int sc0 = static_cast<int>(o.scp & 0xFFu), sc1 = static_cast<int>((o.scp >> 8) & 0xFFu);
    const float sd = fmaf(static_cast<float>(mul24(dot0, sc0)), a.d0, static_cast<float>(mul24(dot1, sc1)) * a.d1);
    const float sm = fmaf(o.m0, a.s0, o.m1 * a.s1);
    return fmaf(o.d, sd, -(o.dmin * sm));
  }

  // dots of one super-block: [dot1 of t = 0..7, sum(qy) of t = 0..7]
  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    int dot0, dot1;
    nibble_dots(o, a, dot0, dot1);
    const int c = (u & 7) >> 1;
    dots[2 * c] += dot0;
    dots[2 * c + 1] += dot1;
    dots[8 + 2 * c] += sum4(a.y0);
    dots[8 + 2 * c + 1] += sum4(a.y1);
  }
};

// ===========================================================================
// Q4_K with one whole 64-weight chunk per lane (the mat-vec and expert
// kernels; the half-chunk layout above serves the many-column kernel's scale
// unpack and the block-dot test kernel's reference layout).
// Unit u: super-block sb = u/4, chunk c = u%4: the 32 code bytes
// qs[32c .. 32c+31] hold sub-blocks t0 = 2c (low nibbles) and t1 = 2c+1
// (high nibbles) whole. A lane loads its super-block's 16-byte header beside
// its two 16-byte code loads, so one header load serves 64 weights, and the
// scale arithmetic of a column dot is shared by 64 weights (32 in the
// half-chunk layout). A wave's 64 lanes read 16 super-blocks' codes.
// ===========================================================================
struct Q4K2 {
  static constexpr int kType = 12, kQK = 256, kBlockBytes = 144;
  static constexpr int kUnitsPerBlock = 4, kDotsPerBlock = 16;

  struct Act {
    uint32_t y0[8], y1[8];   // codes of q8_1 blocks t0 and t1
    float d0, d1;            // their scales
    float s0, s1;            // d8 * (sum of the 32 codes): exact in fp32
  };

  __device__ static void act_blocks(const uint8_t* ycol, int u, const uint8_t*& b0, const uint8_t*& b1) {
    b0 = ycol + static_cast<int64_t>(8 * (u >> 2) + 2 * (u & 3)) * kQ8Bytes;
    b1 = b0 + kQ8Bytes;
  }

  __device__ static int sum8(const uint32_t (&q)[8]) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = bsum4(q[k], s);
    return s;
  }

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const uint8_t *b0, *b1;
    act_blocks(ycol, u, b0, b1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 p0 = ld_x4(b0 + 4 + 16 * h), p1 = ld_x4(b1 + 4 + 16 * h);
      a.y0[4 * h] = p0.x; a.y0[4 * h + 1] = p0.y; a.y0[4 * h + 2] = p0.z; a.y0[4 * h + 3] = p0.w;
      a.y1[4 * h] = p1.x; a.y1[4 * h + 1] = p1.y; a.y1[4 * h + 2] = p1.z; a.y1[4 * h + 3] = p1.w;
    }
    a.d0 = __uint_as_float(ld_u16(b0));
    a.d1 = __uint_as_float(ld_u16(b1));
  }

  __device__ static void finish_act(Act& a) {
    a.d0 = h2f(__float_as_uint(a.d0));
    a.d1 = h2f(__float_as_uint(a.d1));
    a.s0 = a.d0 * static_cast<float>(sum8(a.y0));
    a.s1 = a.d1 * static_cast<float>(sum8(a.y1));
  }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  // fp32 activations: the lane holds both of its q8_1 blocks whole (32
  // values each), so each block's amax needs no exchange with other lanes.
  struct XRaw {
    u32x4 r0[8], r1[8];
  };
  static constexpr int kXWords = 64;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const float* x0 = xcol + static_cast<int64_t>(8 * (u >> 2) + 2 * (u & 3)) * 32;
    const float* x1 = x0 + 32;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x.r0[k] = ld_x4(reinterpret_cast<const uint8_t*>(x0 + 4 * k));
      x.r1[k] = ld_x4(reinterpret_cast<const uint8_t*>(x1 + 4 * k));
    }
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
    float m0 = absmax4(x.r0[0]), m1 = absmax4(x.r1[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      m0 = fmaxf(m0, absmax4(x.r0[k]));
      m1 = fmaxf(m1, absmax4(x.r1[k]));
    }
    const float d0 = q8_scale(m0), d1 = q8_scale(m1);
    int s0 = 0, s1 = 0;
    q8_quant_block(x.r0, d0, a.y0, s0);
    q8_quant_block(x.r1, d1, a.y1, s1);
    a.d0 = q8_d_rounded(d0);
    a.d1 = q8_d_rounded(d1);
    a.s0 = a.d0 * static_cast<float>(s0);
    a.s1 = a.d1 * static_cast<float>(s1);
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int k = 0; k < 8; ++k) { a.y0[k] = 0; a.y1[k] = 0; }
    a.d0 = a.d1 = a.s0 = a.s1 = 0.0f;
  }

  // the half-chunk lane of the chunk's first half: same header offset, the
  // chunk's first code byte, the same scale unpack
  using Lane = Q4K::Lane;
  __device__ static Lane lane(int u) { return Q4K::lane(8 * (u >> 2) + 2 * (u & 3)); }

  struct Wt {
    u32x4 hdr;   // d | dmin, scales[0..3], scales[4..7], scales[8..11]
    u32x4 qs0, qs1;
  };

  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    w.hdr = ld_x4(row + (extra + l.hoff));
    w.qs0 = ld_a16_x4(row + (extra + l.qoff));
    w.qs1 = ld_a16_x4(row + (extra + l.qoff + 16));
  }

  struct Dec {
    uint32_t lo[8], hi[8];   // nibbles of t0 and t1 as unsigned bytes
    uint32_t scp;            // sc of t0 (byte 0) and t1 (byte 1)
    float m0, m1, d, dmin;
  };

  __device__ static void decode(const Wt& w, Dec& o, const Lane& l) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.lo[k] = w.qs0[k] & 0x0F0F0F0Fu;
      o.hi[k] = (w.qs0[k] >> 4) & 0x0F0F0F0Fu;
      o.lo[4 + k] = w.qs1[k] & 0x0F0F0F0Fu;
      o.hi[4 + k] = (w.qs1[k] >> 4) & 0x0F0F0F0Fu;
    }
    o.d = h2f(w.hdr.x);
    o.dmin = h2f(w.hdr.x >> 16);
    uint32_t mp;
    Q4K::chunk_scales(w.hdr, l, o.scp, mp);
    o.m0 = static_cast<float>(mp & 0xFFu);
    o.m1 = static_cast<float>((mp >> 8) & 0xFFu);
  }

  __device__ static void nibble_dots(const Dec& o, const Act& a, int& dot0, int& dot1) {
    dot0 = 0;
    dot1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      dot0 = dot4(o.lo[k], a.y0[k], dot0);
      dot1 = dot4(o.hi[k], a.y1[k], dot1);
    }
  }

  // d * (sc0*d8_0*dot0 + sc1*d8_1*dot1) - dmin * (m0*d8_0*S0 + m1*d8_1*S1)
  __device__ static float col_dot(const Dec& o, const Act& a) {
    int dot0, dot1;
    nibble_dots(o, a, dot0, dot1);
    const int sc0 = static_cast<int>(o.scp & 0xFFu), sc1 = static_cast<int>((o.scp >> 8) & 0xFFu);
    const float sd = fmaf(static_cast<float>(mul24(dot0, sc0)), a.d0, static_cast<float>(mul24(dot1, sc1)) * a.d1);
    const float sm = fmaf(o.m0, a.s0, o.m1 * a.s1);
    return fmaf(o.d, sd, -(o.dmin * sm));
  }

  // dots of one super-block: [dot1 of t = 0..7, sum(qy) of t = 0..7]
  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    int dot0, dot1;
    nibble_dots(o, a, dot0, dot1);
    const int c = u & 3;
    dots[2 * c] += dot0;
    dots[2 * c + 1] += dot1;
    dots[8 + 2 * c] += sum8(a.y0);
    dots[8 + 2 * c + 1] += sum8(a.y1);
  }
};

// ===========================================================================
// Q4_0  [MMVQ §权重的排法, §一次 vec_dot 的解剖]
// 18 bytes: fp16 d @0, qs[16] @2; qs[j] low nibble = element j, high nibble
// = element j+16. Weight = d*(q-8); per block the product is
// d*(d8*sum(q*qy) - 8*s). Unit = one block.
// Blocks are 2-byte aligned: a block at an offset = 2 (mod 4) has its 16
// code bytes dword aligned; one at 0 (mod 4) has them two bytes into a
// dword. Both cases read one dword-aligned 16-byte run plus one 16-bit word,
// all inside the block.
// ===========================================================================
struct Q40 {
  static constexpr int kType = 2, kQK = 32, kBlockBytes = 18;
  static constexpr int kUnitsPerBlock = 1, kDotsPerBlock = 1;

  struct Act {
    uint32_t y[8];
    float d8;
    float s8;      // 8 * s
  };

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const uint8_t* b = ycol + static_cast<int64_t>(u) * kQ8Bytes;
    const u32x4 lo = ld_x4(b + 4), hi = ld_x4(b + 20);
    a.y[0] = lo.x; a.y[1] = lo.y; a.y[2] = lo.z; a.y[3] = lo.w;
    a.y[4] = hi.x; a.y[5] = hi.y; a.y[6] = hi.z; a.y[7] = hi.w;
    a.d8 = __uint_as_float(ld_u32(b));     // fp16 d and s, raw
  }

  __device__ static void finish_act(Act& a) {
    const uint32_t ds = __float_as_uint(a.d8);
    a.d8 = h2f(ds);
    a.s8 = 8.0f * h2f(ds >> 16);
  }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  // fp32 activations: the lane holds its whole q8_1 block.
  struct XRaw {
    u32x4 r[8];
  };
  static constexpr int kXWords = 32;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const float* p = xcol + static_cast<int64_t>(u) * 32;
#pragma unroll
    for (int k = 0; k < 8; ++k) x.r[k] = ld_x4(reinterpret_cast<const uint8_t*>(p + 4 * k));
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
    float m = absmax4(x.r[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) m = fmaxf(m, absmax4(x.r[k]));
    const float d = q8_scale(m);
    int sq = 0;
    q8_quant_block(x.r, d, a.y, sq);
    a.d8 = q8_d_rounded(d);
    a.s8 = 8.0f * h2f(f2h_bits(q8_s(d, sq)));
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a.y[k] = 0;
    a.d8 = a.s8 = 0.0f;
  }

  struct Lane {
    uint32_t off;    // block offset from the row start
  };
  __device__ static Lane lane(int u) { return Lane{static_cast<uint32_t>(u * kBlockBytes)}; }

  struct Wt {
    u32x4 run;       // dword-aligned 16 bytes
    uint32_t extra;  // 16-bit word: d (odd placement) or qs[14..15]
    bool odd;        // block address = 2 (mod 4)
  };

  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t off = extra + l.off;
    w.odd = ((static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row)) + off) & 2u) != 0;
    w.run = ld_x4(row + (off + (w.odd ? 2u : 0u)));
    w.extra = ld_u16(row + (off + (w.odd ? 0u : 16u)));
  }

  struct Dec {
    uint32_t lo[4], hi[4];
    float d;
  };

  __device__ static void decode(const Wt& w, Dec& o, const Lane&) {
    uint32_t qs[4];
    qs[0] = w.odd ? w.run.x : shr16_pair(w.run.y, w.run.x);
    qs[1] = w.odd ? w.run.y : shr16_pair(w.run.z, w.run.y);
    qs[2] = w.odd ? w.run.z : shr16_pair(w.run.w, w.run.z);
    qs[3] = w.odd ? w.run.w : shr16_pair(w.extra, w.run.w);
    o.d = h2f(w.odd ? w.extra : w.run.x);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.lo[k] = qs[k] & 0x0F0F0F0Fu;
      o.hi[k] = (qs[k] >> 4) & 0x0F0F0F0Fu;
    }
  }

  __device__ static int isum(const Dec& o, const Act& a) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) s = dot4(o.lo[k], a.y[k], s);
#pragma unroll
    for (int k = 0; k < 4; ++k) s = dot4(o.hi[k], a.y[4 + k], s);
    return s;
  }

  __device__ static float col_dot(const Dec& o, const Act& a) {
    return o.d * fmaf(a.d8, static_cast<float>(isum(o, a)), -a.s8);
  }

  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    dots[0] += isum(o, a);
  }
};

// ===========================================================================
// Q8_0  [LLM §量化格式 (34 bytes per 32 weights); MMVQ §权重的排法]
// 34 bytes: fp16 d @0, int8 qs[32] @2 (element e = byte 2+e). Weight = d*q;
// per block the product is d*d8*sum(q*qy) (symmetric: no s term). Unit =
// one block. Blocks are 2-byte aligned: at an offset = 2 (mod 4) the 32 code
// bytes are dword aligned (two 16-byte runs) and d is the 16-bit word before
// them; at 0 (mod 4) the block is read as two 16-byte runs from its start
// plus its last 16-bit word, and the codes are re-aligned by two bytes.
// ===========================================================================
struct Q80 {
  static constexpr int kType = 8, kQK = 32, kBlockBytes = 34;
  static constexpr int kUnitsPerBlock = 1, kDotsPerBlock = 1;

  struct Act {
    uint32_t y[8];
    float d8;
  };

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const uint8_t* b = ycol + static_cast<int64_t>(u) * kQ8Bytes;
    const u32x4 lo = ld_x4(b + 4), hi = ld_x4(b + 20);
    a.y[0] = lo.x; a.y[1] = lo.y; a.y[2] = lo.z; a.y[3] = lo.w;
    a.y[4] = hi.x; a.y[5] = hi.y; a.y[6] = hi.z; a.y[7] = hi.w;
    a.d8 = __uint_as_float(ld_u16(b));      // fp16 d, raw
  }

  __device__ static void finish_act(Act& a) { a.d8 = h2f(__float_as_uint(a.d8)); }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  // fp32 activations: the lane holds its whole q8_1 block.
  struct XRaw {
    u32x4 r[8];
  };
  static constexpr int kXWords = 32;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const float* p = xcol + static_cast<int64_t>(u) * 32;
#pragma unroll
    for (int k = 0; k < 8; ++k) x.r[k] = ld_x4(reinterpret_cast<const uint8_t*>(p + 4 * k));
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
    float m = absmax4(x.r[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) m = fmaxf(m, absmax4(x.r[k]));
    const float d = q8_scale(m);
    int sq = 0;
    q8_quant_block(x.r, d, a.y, sq);
    a.d8 = q8_d_rounded(d);
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a.y[k] = 0;
    a.d8 = 0.0f;
  }

  struct Lane {
    uint32_t off;    // block offset from the row start
  };
  __device__ static Lane lane(int u) { return Lane{static_cast<uint32_t>(u * kBlockBytes)}; }

  struct Wt {
    u32x4 lo, hi;    // two dword-aligned 16-byte runs
    uint32_t extra;  // 16-bit word: d (offset 2 mod 4) or code bytes 30..31
    bool odd;        // block address = 2 (mod 4)
  };

  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t off = extra + l.off;
    w.odd = ((static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row)) + off) & 2u) != 0;
    const uint32_t run = off + (w.odd ? 2u : 0u);
    w.lo = ld_x4(row + run);
    w.hi = ld_x4(row + (run + 16u));
    w.extra = ld_u16(row + (off + (w.odd ? 0u : 32u)));
  }

  struct Dec {
    uint32_t q[8];
    float d;
  };

  __device__ static void decode(const Wt& w, Dec& o, const Lane&) {
    const uint32_t dw[9] = {w.lo.x, w.lo.y, w.lo.z, w.lo.w, w.hi.x, w.hi.y, w.hi.z, w.hi.w, w.extra};
#pragma unroll
    for (int k = 0; k < 8; ++k) o.q[k] = w.odd ? dw[k] : shr16_pair(dw[k + 1], dw[k]);
    o.d = h2f(w.odd ? w.extra : w.lo.x);
  }

  __device__ static int isum(const Dec& o, const Act& a) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = dot4(o.q[k], a.y[k], s);
    return s;
  }

  __device__ static float col_dot(const Dec& o, const Act& a) {
    return o.d * (a.d8 * static_cast<float>(isum(o, a)));
  }

  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    dots[0] += isum(o, a);
  }
};

// ===========================================================================
// Q6_K  [MMVQ §dp4a, §一次 vec_dot 的解剖]
// 210 bytes: ql[128] @0 (low 4 bits), qh[64] @128 (high 2 bits), int8
// sc[16] @192, fp16 d @208. Element 128h + 32g + l (h 0..1, g 0..3, l 0..31):
// low bits from ql[64h + 32(g%2) + l] (low nibble for g < 2, high nibble
// otherwise), high bits (qh[32h + l] >> 2g) & 3; sub-block 8h + 2g + l/16;
// weight = d*sc*(q-32).
// Unit u: super-block sb = u/4, h = (u/2)%2, lq = u%2 (l in 16lq..16lq+15):
// pieces A = ql[64h+16lq ..+16], B = ql[64h+32+16lq ..+16],
// C = qh[32h+16lq ..+16]; sub-blocks 8h + 2g + lq for g = 0..3, each paired
// with q8_1 block 8sb + 4h + g, codes 16lq..16lq+15.
// Blocks are 2-byte aligned: a piece at an address = 2 (mod 4) is read as
// the dword-aligned run starting two bytes into it plus its first 16-bit
// word, then re-aligned (all reads stay inside the super-block).
// ===========================================================================
struct Q6K {
  static constexpr int kType = 14, kQK = 256, kBlockBytes = 210;
  static constexpr int kUnitsPerBlock = 4, kDotsPerBlock = 16;

  struct Act {
    uint32_t y[4][4];
    float d8[4];
    int c32[4];      // 32 * (sum of the 16 codes): the -32 offset term
  };

  __device__ static const uint8_t* act_block(const uint8_t* ycol, int u, int g) {
    const int sb = u >> 2, h = (u >> 1) & 1;
    return ycol + static_cast<int64_t>(8 * sb + 4 * h + g) * kQ8Bytes;
  }

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const int lq = u & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint8_t* b = act_block(ycol, u, g);
      const u32x4 q = ld_x4(b + 4 + 16 * lq);
      a.y[g][0] = q.x; a.y[g][1] = q.y; a.y[g][2] = q.z; a.y[g][3] = q.w;
      a.d8[g] = __uint_as_float(ld_u16(b));
    }
  }

  __device__ static void finish_act(Act& a) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      a.d8[g] = h2f(__float_as_uint(a.d8[g]));
      a.c32[g] = 32 * bsum4(a.y[g][3], bsum4(a.y[g][2], bsum4(a.y[g][1], bsum4(a.y[g][0], 0))));
    }
  }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  // fp32 activations: for each g the lane holds half of q8_1 block
  // 8sb+4h+g (16 values); the lane next to it (unit u ^ 1, the other lq)
  // holds the other half.
  struct XRaw {
    u32x4 r[4][4];
  };
  static constexpr int kXWords = 64;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const int sb = u >> 2, h = (u >> 1) & 1, lq = u & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float* p = xcol + static_cast<int64_t>(8 * sb + 4 * h + g) * 32 + 16 * lq;
#pragma unroll
      for (int k = 0; k < 4; ++k) x.r[g][k] = ld_x4(reinterpret_cast<const uint8_t*>(p + 4 * k));
    }
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float m = absmax4(x.r[g][0]);
#pragma unroll
      for (int k = 1; k < 4; ++k) m = fmaxf(m, absmax4(x.r[g][k]));
      const float d = q8_scale(max_with_pair(m));
      int sq = 0;
      q8_quant_block(x.r[g], d, a.y[g], sq);
      a.d8[g] = q8_d_rounded(d);
      a.c32[g] = 32 * sq;
    }
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int k = 0; k < 4; ++k) a.y[g][k] = 0;
      a.d8[g] = 0.0f;
      a.c32[g] = 0;
    }
  }

  struct Lane {
    uint32_t blk;                 // super-block offset from the row start
    uint32_t oA, oB, oC, oS;      // piece offsets inside the super-block
    uint32_t lq;
  };
  __device__ static Lane lane(int u) {
    Lane l;
    const int sb = u >> 2, h = (u >> 1) & 1, lq = u & 1;
    l.blk = static_cast<uint32_t>(sb * kBlockBytes);
    l.oA = 64 * h + 16 * lq;
    l.oB = l.oA + 32;
    l.oC = 128 + 32 * h + 16 * lq;
    l.oS = 192 + 8 * h;
    l.lq = lq;
    return l;
  }

  // Pieces start at even offsets. When a piece's address is 2 (mod 4) the
  // lane reads the dword-aligned run starting two bytes INTO the piece plus
  // the piece's first 16-bit word, so every offset is at or above the
  // piece start and every byte read lies inside the super-block.
  struct Wt {
    u32x4 A, B, C;              // dword-aligned runs
    uint32_t a0, b0, c0;        // first 16-bit word of each piece
    u32x2 S;                    // dword-aligned run over the 8 scales
    uint32_t s0;                // first 16-bit word of the scales
    uint32_t dbits;
    bool odd;
  };

  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t blk = extra + l.blk;
    w.odd = ((static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row)) + blk) & 2u) != 0;
    const uint32_t sh = w.odd ? 2u : 0u;
    w.A = ld_x4(row + (blk + l.oA + sh));
    w.B = ld_x4(row + (blk + l.oB + sh));
    w.C = ld_x4(row + (blk + l.oC + sh));
    w.S = ld_x2(row + (blk + l.oS + sh));
    w.a0 = ld_u16(row + (blk + l.oA));
    w.b0 = ld_u16(row + (blk + l.oB));
    w.c0 = ld_u16(row + (blk + l.oC));
    w.s0 = ld_u16(row + (blk + l.oS));
    w.dbits = ld_u16(row + (blk + 208));
  }

  struct Dec {
    uint32_t code[4][4];        // 6-bit codes, 4 per word, sub-block g
    int sc[4];
    float d;
  };

  // 16 piece bytes from a run read two bytes into the piece (odd) or at it
  __device__ static void realign(const u32x4& r, uint32_t head, bool odd, uint32_t (&o)[4]) {
    o[0] = odd ? ((r.x << 16) | (head & 0xFFFFu)) : r.x;
    o[1] = odd ? shr16_pair(r.y, r.x) : r.y;
    o[2] = odd ? shr16_pair(r.z, r.y) : r.z;
    o[3] = odd ? shr16_pair(r.w, r.z) : r.w;
  }

  __device__ static void decode(const Wt& w, Dec& o, const Lane& l) {
    uint32_t A[4], B[4], C[4];
    realign(w.A, w.a0, w.odd, A);
    realign(w.B, w.b0, w.odd, B);
    realign(w.C, w.c0, w.odd, C);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.code[0][k] = (A[k] & 0x0F0F0F0Fu) | ((C[k] << 4) & 0x30303030u);
      o.code[1][k] = (B[k] & 0x0F0F0F0Fu) | ((C[k] << 2) & 0x30303030u);
      o.code[2][k] = ((A[k] >> 4) & 0x0F0F0F0Fu) | (C[k] & 0x30303030u);
      o.code[3][k] = ((B[k] >> 4) & 0x0F0F0F0Fu) | ((C[k] >> 2) & 0x30303030u);
    }
    const uint32_t s0 = w.odd ? ((w.S.x << 16) | (w.s0 & 0xFFFFu)) : w.S.x;   // scales 8h+0..3
    const uint32_t s1 = w.odd ? shr16_pair(w.S.y, w.S.x) : w.S.y;              // scales 8h+4..7
    o.sc[0] = sbfe(s0, 8 * l.lq, 8);
    o.sc[1] = sbfe(s0, 8 * l.lq + 16, 8);
    o.sc[2] = sbfe(s1, 8 * l.lq, 8);
    o.sc[3] = sbfe(s1, 8 * l.lq + 16, 8);
    o.d = h2f(w.dbits);
  }

  __device__ static int isum(const Dec& o, const Act& a, int g) {
    int s = -a.c32[g];
#pragma unroll
    for (int k = 0; k < 4; ++k) s = dot4(o.code[g][k], a.y[g][k], s);
    return s;
  }

  __device__ static float col_dot(const Dec& o, const Act& a) {
    float acc = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) acc = fmaf(static_cast<float>(mul24(isum(o, a, g), o.sc[g])), a.d8[g], acc);
    return o.d * acc;
  }

  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    const int h = (u >> 1) & 1, lq = u & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) dots[8 * h + 2 * g + lq] += isum(o, a, g);
  }
};

// ===========================================================================
// Old-style 32-weight blocks with an offset term: Q4_1, Q5_0, Q5_1
// [MMVQ §权重的排法 (old-style blocks, Q5_1 named among them), §激活的量化;
// GGUF16 §16.1.1 (type ids 3, 6, 7)]. The pages name these formats without
// their layouts; the layouts are the published GGUF block definitions:
//   Q4_1: fp16 d @0, fp16 m @2, qs[16] @4 (20 bytes); weight d*q + m
//   Q5_0: fp16 d @0, qh[4] @2, qs[16] @6 (22 bytes); weight d*(q - 16)
//   Q5_1: fp16 d @0, fp16 m @2, qh[4] @4, qs[16] @8 (24 bytes); weight d*q + m
// Low 4 bits as in Q4_0 (low nibble of qs[j] = element j, high nibble =
// element j+16); bit e of the little-endian qh word is bit 4 of element e.
// Per block: d*d8*sum(q*qy) plus the offset term from the q8_1 block's s
// (m*s, or -16*d*s for Q5_0), as Q4_0 takes its zero point from s. Unit =
// one block; the activation side is Q4_0's with s kept unscaled.
// ===========================================================================
struct Legacy32Act {
  static constexpr int kQK = 32, kUnitsPerBlock = 1, kDotsPerBlock = 1;

  struct Act {
    uint32_t y[8];
    float d8;
    float s;
  };

  __device__ static void issue_act(Act& a, const uint8_t* ycol, int u) {
    const uint8_t* b = ycol + static_cast<int64_t>(u) * kQ8Bytes;
    const u32x4 lo = ld_x4(b + 4), hi = ld_x4(b + 20);
    a.y[0] = lo.x; a.y[1] = lo.y; a.y[2] = lo.z; a.y[3] = lo.w;
    a.y[4] = hi.x; a.y[5] = hi.y; a.y[6] = hi.z; a.y[7] = hi.w;
    a.d8 = __uint_as_float(ld_u32(b));     // fp16 d and s, raw
  }

  __device__ static void finish_act(Act& a) {
    const uint32_t ds = __float_as_uint(a.d8);
    a.d8 = h2f(ds);
    a.s = h2f(ds >> 16);
  }

  __device__ static void load_act(Act& a, const uint8_t* ycol, int u) {
    issue_act(a, ycol, u);
    finish_act(a);
  }

  struct XRaw {
    u32x4 r[8];
  };
  static constexpr int kXWords = 32;

  __device__ static void load_x(XRaw& x, const float* xcol, int u) {
    const float* p = xcol + static_cast<int64_t>(u) * 32;
#pragma unroll
    for (int k = 0; k < 8; ++k) x.r[k] = ld_x4(reinterpret_cast<const uint8_t*>(p + 4 * k));
  }

  __device__ static void quant_x(Act& a, const XRaw& x) {
    float m = absmax4(x.r[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) m = fmaxf(m, absmax4(x.r[k]));
    const float d = q8_scale(m);
    int sq = 0;
    q8_quant_block(x.r, d, a.y, sq);
    a.d8 = q8_d_rounded(d);
    a.s = h2f(f2h_bits(q8_s(d, sq)));
  }

  __device__ static void zero_act(Act& a) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a.y[k] = 0;
    a.d8 = a.s = 0.0f;
  }

  struct Lane {
    uint32_t off;    // block offset from the row start
  };

  // the 8 code words: lo[k] elements 4k..4k+3, hi[k] elements 16+4k.. (one
  // byte each), with bit 4 from qh (the 4 qh bits of a word spread to the
  // bytes' bit 4 by a multiply: bit i of b lands at bit 8i)
  struct Dec {
    uint32_t lo[4], hi[4];
    float d, off;    // off: m, or -16*d
  };

  __device__ static uint32_t spread4(uint32_t qh, int first) {
    const uint32_t b = (qh >> first) & 0xFu;
    return ((b * 0x00204081u) & 0x01010101u) << 4;
  }

  __device__ static void split(const uint32_t (&qs)[4], uint32_t qh, bool five, Dec& o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.lo[k] = qs[k] & 0x0F0F0F0Fu;
      o.hi[k] = (qs[k] >> 4) & 0x0F0F0F0Fu;
      if (five) {
        o.lo[k] |= spread4(qh, 4 * k);
        o.hi[k] |= spread4(qh, 16 + 4 * k);
      }
    }
  }

  __device__ static int isum(const Dec& o, const Act& a) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) s = dot4(o.lo[k], a.y[k], s);
#pragma unroll
    for (int k = 0; k < 4; ++k) s = dot4(o.hi[k], a.y[4 + k], s);
    return s;
  }

  // d*d8*isum + off*s
  __device__ static float col_dot(const Dec& o, const Act& a) {
    return fmaf(o.d * a.d8, static_cast<float>(isum(o, a)), o.off * a.s);
  }

  __device__ static void int_dots(const Dec& o, const uint8_t* ycol, int u, int* dots) {
    Act a;
    load_act(a, ycol, u);
    dots[0] += isum(o, a);
  }
};

// Q4_1: 20-byte blocks, 4-byte aligned (rows of K/32 blocks from a 16-byte
// aligned base): d | m as one word, the 16 code bytes as one run.
struct Q41 : Legacy32Act {
  static constexpr int kType = 3, kBlockBytes = 20;
  __device__ static Lane lane(int u) { return Lane{static_cast<uint32_t>(u * kBlockBytes)}; }
  struct Wt {
    u32x4 qs;
    uint32_t dm;
  };
  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t off = extra + l.off;
    w.dm = ld_u32(row + off);
    w.qs = ld_x4(row + (off + 4));
  }
  __device__ static void decode(const Wt& w, Dec& o, const Lane&) {
    const uint32_t qs[4] = {w.qs.x, w.qs.y, w.qs.z, w.qs.w};
    split(qs, 0u, false, o);
    o.d = h2f(w.dm);
    o.off = h2f(w.dm >> 16);
  }
};

// Q5_1: 24-byte blocks, 8-byte aligned: d | m, qh, then the codes.
struct Q51 : Legacy32Act {
  static constexpr int kType = 7, kBlockBytes = 24;
  __device__ static Lane lane(int u) { return Lane{static_cast<uint32_t>(u * kBlockBytes)}; }
  struct Wt {
    u32x4 qs;
    uint32_t dm, qh;
  };
  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t off = extra + l.off;
    const u32x2 h = ld_x2(row + off);
    w.dm = h.x;
    w.qh = h.y;
    w.qs = ld_x4(row + (off + 8));
  }
  __device__ static void decode(const Wt& w, Dec& o, const Lane&) {
    const uint32_t qs[4] = {w.qs.x, w.qs.y, w.qs.z, w.qs.w};
    split(qs, w.qh, true, o);
    o.d = h2f(w.dm);
    o.off = h2f(w.dm >> 16);
  }
};

// Q5_0: 22-byte blocks, only 2-byte aligned. Every read stays inside the
// block: at an offset = 0 (mod 4) a 16-byte run from the start, the word at
// 16 and the 16-bit word at 20; at 2 (mod 4) the 16-bit d, a 16-byte run from
// byte 2 and the word at 18.
struct Q50 : Legacy32Act {
  static constexpr int kType = 6, kBlockBytes = 22;
  __device__ static Lane lane(int u) { return Lane{static_cast<uint32_t>(u * kBlockBytes)}; }
  struct Wt {
    u32x4 run;
    uint32_t w1, w2;
    bool odd;        // block address = 2 (mod 4)
  };
  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    const uint32_t off = extra + l.off;
    w.odd = ((static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row)) + off) & 2u) != 0;
    w.run = ld_x4(row + (off + (w.odd ? 2u : 0u)));
    w.w1 = ld_u32(row + (off + (w.odd ? 18u : 16u)));
    w.w2 = ld_u16(row + (off + (w.odd ? 0u : 20u)));
  }
  __device__ static void decode(const Wt& w, Dec& o, const Lane&) {
    // odd: d = w2, bytes 2..17 = run, 18..21 = w1
    // even: bytes 0..15 = run, 16..19 = w1, 20..21 = w2
    const uint32_t qh = w.odd ? w.run.x : shr16_pair(w.run.y, w.run.x);
    uint32_t qs[4];
    qs[0] = w.odd ? w.run.y : shr16_pair(w.run.z, w.run.y);
    qs[1] = w.odd ? w.run.z : shr16_pair(w.run.w, w.run.z);
    qs[2] = w.odd ? w.run.w : shr16_pair(w.w1, w.run.w);
    qs[3] = w.odd ? w.w1 : shr16_pair(w.w2, w.w1);
    split(qs, qh, true, o);
    o.d = h2f(w.odd ? w.w2 : w.run.x);
    o.off = -16.0f * o.d;
  }
};

// ===========================================================================
// Q5_K [MMVQ §激活的量化 (a min-term format); GGUF16 §16.1.1 (type id 13)].
// The layout is the published GGUF block definition (the pages do not print
// it): fp16 d @0, fp16 dmin @2, the 12 packed scale/min bytes of Q4_K @4,
// qh[32] @16, qs[128] @48; 176 bytes. Element l of the low (high) nibble run
// of 64-element chunk c is in sub-block t = 2c (2c + 1) and takes bit t of
// qh[l] as bit 4. Weight d*sc_t*q - dmin*m_t, q in 0..31; the dot is Q4_K's.
// Unit as Q4_K's half chunks: 16 code bytes of chunk c, half h (elements
// l = 16h .. 16h+15 of sub-blocks 2c and 2c+1), plus the header and the 16
// qh bytes of those elements.
// ===========================================================================
struct Q5K : Q4K {
  static constexpr int kType = 13, kBlockBytes = 176;
  struct Lane : Q4K::Lane {
    uint32_t qhoff;
    uint32_t t0;     // sub-block of the low nibbles (2c)
  };
  __device__ static Lane lane(int u) {
    Lane l;
    const int sb = u >> 3, p = u & 7, c = p >> 1, half = p & 1;
    l.hoff = static_cast<uint32_t>(sb * kBlockBytes);
    l.qoff = l.hoff + 48 + 16 * p;
    l.qhoff = l.hoff + 16 + 16 * half;
    l.t0 = static_cast<uint32_t>(2 * c);
    l.lo = c < 2;
    l.sh = 16u * (c & 1);
    l.shm = l.lo ? l.sh : l.sh + 4;
    l.maskA = l.lo ? 0x3F3Fu : 0x0F0Fu;
    l.maskB = l.lo ? 0u : 0x3030u;
    return l;
  }
  struct Wt {
    u32x4 qs, hdr, qh;
  };
  __device__ static void load_wt(Wt& w, const uint8_t* row, uint32_t extra, const Lane& l) {
    w.hdr = ld_x4(row + (extra + l.hoff));
    w.qs = ld_a16_x4(row + (extra + l.qoff));
    w.qh = ld_a16_x4(row + (extra + l.qhoff));
  }
  __device__ static void decode(const Wt& w, Dec& o, const Lane& l) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o.lo[k] = (w.qs[k] & 0x0F0F0F0Fu) | (((w.qh[k] >> l.t0) & 0x01010101u) << 4);
      o.hi[k] = ((w.qs[k] >> 4) & 0x0F0F0F0Fu) | (((w.qh[k] >> (l.t0 + 1)) & 0x01010101u) << 4);
    }
    o.d = h2f(w.hdr.x);
    o.dmin = h2f(w.hdr.x >> 16);
    uint32_t mp;
    chunk_scales(w.hdr, l, o.scp, mp);
    o.m0 = static_cast<float>(mp & 0xFFu);
    o.m1 = static_cast<float>((mp >> 8) & 0xFFu);
  }
};

}  // namespace qmv
