// q8.hpp - q8_1 quantization arithmetic, shared by the stand-alone
// quantizer kernel and the fused (fp32-input) mat-vec prologue, so both
// produce the same codes and scales bit for bit.
//
// [MMVQ §激活的量化] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时一条
// 量化权重如何被 dp4a 逐块点积", section 激活的量化: per block of 32 values,
// d = amax/127 in fp32, q = roundf(x/d) (0 when d == 0), s = d*sum(q); d and s
// are stored as fp16 (round to nearest even).
#pragma once

#include <math.h>

#include "common.hpp"

namespace qmv {

// fp32 scale of a block from its amax (IEEE division: hipcc's default
// correctly rounded fp32 division, and fp32 denormals kept).
__device__ __forceinline__ float q8_scale(float amax) { return amax / 127.0f; }

// One code; a zero scale (amax == 0, or amax/127 underflowing) gives 0.
// Branch-free: the quotient is formed against a divisor of 1 when d == 0
// (then every x of the block is 0 or tiny, so the unused quotient stays in
// int range) and the result selected, so the 32 codes of a block are
// straight-line code rather than one branch each.
__device__ __forceinline__ int q8_code(float x, float d) {
  const bool z = d == 0.0f;
  const int q = static_cast<int>(roundf(x / (z ? 1.0f : d)));
  return z ? 0 : q;
}

__device__ __forceinline__ float absmax4(const u32x4& r) {
  return fmaxf(fmaxf(fabsf(__uint_as_float(r.x)), fabsf(__uint_as_float(r.y))),
               fmaxf(fabsf(__uint_as_float(r.z)), fabsf(__uint_as_float(r.w))));
}

// Codes of four fp32 values packed in one word (byte k = value k); their sum
// is added to `sum`.
__device__ __forceinline__ uint32_t q8_quant4(const u32x4& r, float d, int& sum) {
  const int q0 = q8_code(__uint_as_float(r.x), d), q1 = q8_code(__uint_as_float(r.y), d);
  const int q2 = q8_code(__uint_as_float(r.z), d), q3 = q8_code(__uint_as_float(r.w), d);
  sum += q0 + q1 + q2 + q3;
  return (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | (static_cast<uint32_t>(q3) << 24);
}

// Low bytes of four words packed into one word (byte k = low byte of w_k).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
#ifndef QMV_HOST_MODEL
  // v_perm_b32 selects bytes of {hi, lo}: 0x0c yields 0
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x04000c0cu);
  return lo | hi;
#else
  return (w0 & 0xFFu) | ((w1 & 0xFFu) << 8) | ((w2 & 0xFFu) << 16) | ((w3 & 0xFFu) << 24);
#endif
}

// Codes of the 4*W values of one q8_1 block that the lane holds (word k of
// `out` packs the codes of v[k]), their sum added to `sum`; equal to
// q8_quant4 on every word, at about a quarter of the arithmetic:
//   r = 1/d correctly rounded, once per block; p = x*r (exact product).
//   With u = 2^-24, |p - x/d| <= u*|x/d| (the rounding of r) and
//   |RN(x/d) - x/d| <= u*|x/d|, where |x/d| <= 127.0000076 since |x| <= amax
//   and d = RN(amax/127): so |p - RN(x/d)| <= 254.00002*u < 2^-16 - 2^-25.
//   One fma rounds p to an integer (adding 1.5*2^23, whose ulp is 1: ties to
//   even), the bias comes off exactly, and a second fma gives p minus that
//   integer with an error of at most 2^-25. When that residue is below
//   1/2 - 2^-16, RN(x/d) lies strictly inside the same unit interval around
//   the integer, which is then round(RN(x/d)) (no tie can occur), and its
//   two's complement low byte is the low byte of the biased sum. Otherwise
//   (about 2^-15 of the values), or when d is 0 or subnormal (r out of
//   range), the block is redone with exact quotients.
template <int W>
__device__ __forceinline__ void q8_quant_block(const u32x4 (&v)[W], float d, uint32_t (&out)[W], int& sum) {
  constexpr float kBias = 0x1.8p23f;
  const bool normal = d >= 0x1p-126f;
  const float r = 1.0f / (normal ? d : 1.0f);
  bool near = !normal;
  int s = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    uint32_t m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __uint_as_float(v[k][e]);
      const float biased = fmaf(x, r, kBias);          // x*r rounded to an integer, biased
      const float rq = biased - kBias;                 // that integer, exact
      near = near || fabsf(fmaf(x, r, -rq)) >= 0.5f - 0x1p-16f;
      m[e] = __float_as_uint(biased);
    }
    out[k] = pack_low_bytes(m[0], m[1], m[2], m[3]);
    s = dot4(out[k], 0x01010101u, s);
  }
  if (near) {
    s = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) out[k] = q8_quant4(v[k], d, s);
  }
  sum += s;
}

__device__ __forceinline__ uint32_t f2h_bits(float v) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v)));
}

// The stored (fp16) value of d, as a float: what the mat-vec multiplies by.
__device__ __forceinline__ float q8_d_rounded(float d) { return h2f(f2h_bits(d)); }

// s = d*sum(q) as an fp32 product. The empty asm pins the fp32 result in a
// register: without it the multiply and the later f16 conversion fuse into
// one v_fma_mixlo_f16, which rounds once instead of twice.
__device__ __forceinline__ float q8_s(float d, int sumq) {
  float s = d * static_cast<float>(sumq);
#ifndef QMV_HOST_MODEL
  asm volatile("" : "+v"(s));
#endif
  return s;
}

// Cross-lane maximum with the neighbour lane (lane ^ 1): the two lanes that
// hold the two halves of one 32-value block.
__device__ __forceinline__ float max_with_pair(float v) {
#ifndef QMV_HOST_MODEL
  return fmaxf(v, dpp_f<kDppXor1>(v));
#else
  return v;
#endif
}

}  // namespace qmv
