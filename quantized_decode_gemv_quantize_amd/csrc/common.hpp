// common.hpp - device helpers shared by the MMVQ kernels (gfx950, wave64).
//
// Cross-lane reduction, raw loads and small integer helpers. Everything here
// is CDNA4 code: 64-lane wavefronts, DPP row/quad permutes, and the gfx950
// v_permlane16_swap / v_permlane32_swap instructions.
//
// With QMV_HOST_MODEL defined (a host-only clang build used by the test
// suite), the loads become bounds-checked host reads that record every
// access outside the registered buffers, and the few integer builtins the
// block decoders use get portable equivalents; the cross-lane part is left
// out. This lets the host run the exact addressing code of the kernels.
#pragma once

#include <stdint.h>

#ifndef QMV_HOST_MODEL
#include <hip/hip_runtime.h>
#else
#include <string.h>
#include <vector>
#define __device__
#define __host__
#define __forceinline__ inline
#endif

namespace qmv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxCols = 8;
constexpr int kMaxThreads = 1024;
constexpr int kLaunchBound = 512;       // 8 waves per workgroup at most
constexpr int kMaxWavesPerBlock = kLaunchBound / kWave;

#ifdef QMV_HOST_MODEL
namespace hostmodel {
struct Range {
  const uint8_t* lo;
  const uint8_t* hi;
};
inline std::vector<Range>& ranges() {
  static std::vector<Range> r;
  return r;
}
inline long& violations() {
  static long v = 0;
  return v;
}
inline long& accesses() {
  static long v = 0;
  return v;
}
// True if [p, p+n) lies inside one registered buffer and p is aligned as the
// device load requires; otherwise counts a violation (and nothing is read).
inline bool ok(const uint8_t* p, size_t n, uintptr_t align) {
  ++accesses();
  if (reinterpret_cast<uintptr_t>(p) % align != 0) { ++violations(); return false; }
  for (const Range& r : ranges())
    if (p >= r.lo && p + n <= r.hi) return true;
  ++violations();
  return false;
}
}  // namespace hostmodel

inline u32x4 ld_a16_x4(const uint8_t* p) {
  u32x4 v = {0, 0, 0, 0};
  if (hostmodel::ok(p, 16, 16)) memcpy(&v, p, 16);
  return v;
}
inline u32x4 ld_x4(const uint8_t* p) {
  u32x4 v = {0, 0, 0, 0};
  if (hostmodel::ok(p, 16, 4)) memcpy(&v, p, 16);
  return v;
}
inline u32x2 ld_x2(const uint8_t* p) {
  u32x2 v = {0, 0};
  if (hostmodel::ok(p, 8, 4)) memcpy(&v, p, 8);
  return v;
}
inline uint32_t ld_u16(const uint8_t* p) {
  uint16_t v = 0;
  if (hostmodel::ok(p, 2, 2)) memcpy(&v, p, 2);
  return v;
}
inline uint32_t ld_u32(const uint8_t* p) {
  uint32_t v = 0;
  if (hostmodel::ok(p, 4, 4)) memcpy(&v, p, 4);
  return v;
}
inline uint32_t shr16_pair(uint32_t hi, uint32_t lo) {
  return static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> 16);
}
inline int dot4(uint32_t a, uint32_t b, int c) {
  for (int k = 0; k < 4; ++k)
    c += static_cast<int8_t>(a >> (8 * k)) * static_cast<int8_t>(b >> (8 * k));
  return c;
}
inline int mul24(int a, int b) { return a * b; }
inline float __uint_as_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
inline uint32_t __float_as_uint(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
inline int sbfe(uint32_t v, uint32_t off, uint32_t width) {
  return static_cast<int>(v << (32 - off - width)) >> (32 - width);
}
#else

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// ---------------------------------------------------------------------------
// Loads. Ordinary cached loads throughout: the streaming (non-temporal) hint
// measured slower for the weight stream, whose header and code bytes share
// cache lines.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_a16_x4(const uint8_t* p) {  // p 16-byte aligned
  return *reinterpret_cast<const u32x4*>(__builtin_assume_aligned(p, 16));
}
__device__ __forceinline__ u32x4 ld_x4(const uint8_t* p) {      // p 4-byte aligned
  const uint32_t* q = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  u32x4 v;
  __builtin_memcpy(&v, q, 16);
  return v;
}
__device__ __forceinline__ u32x2 ld_x2(const uint8_t* p) {      // p 4-byte aligned
  const uint32_t* q = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  u32x2 v;
  __builtin_memcpy(&v, q, 8);
  return v;
}
__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {   // p 2-byte aligned
  return *reinterpret_cast<const uint16_t*>(__builtin_assume_aligned(p, 2));
}
__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {   // p 4-byte aligned
  return *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
}

// ({hi, lo} >> 16) as 32 bits: re-aligns a 16-byte run that starts two bytes
// into a dword.
__device__ __forceinline__ uint32_t shr16_pair(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// 4-way signed int8 dot product with accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// 24-bit signed multiply (v_mul_i32_i24); both factors fit in 24 bits here.
__device__ __forceinline__ int mul24(int a, int b) { return __mul24(a, b); }

// Signed bit-field extract (v_bfe_i32).
__device__ __forceinline__ int sbfe(uint32_t v, uint32_t off, uint32_t width) {
  return __builtin_amdgcn_sbfe(v, off, width);
}
#endif

// fp16 bit pattern (low 16 bits) -> float.
__device__ __forceinline__ float h2f(uint32_t bits) {
  _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu));
  return static_cast<float>(h);
}

constexpr int pow2ceil(int v) { int p = 1; while (p < v) p <<= 1; return p; }

// Lambdas of the kernel bodies are inlined like the __forceinline__
// functions around them (a lambda the inliner leaves out of line takes its
// captured register arrays through scratch memory).
#define QMV_INLINE __attribute__((always_inline))

// f(Idx<0>{}), ..., f(Idx<N-1>{}): a loop whose index is a compile-time
// constant in the body, for bodies too large for the loop unroller (a
// runtime index into a register array puts the array in scratch memory).
template <int I>
struct Idx {
  static constexpr int value = I;
};
template <int I, int N, class Fn>
__host__ __device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(Idx<I>{});
    static_for<I + 1, N>(f);
  }
}

#ifndef QMV_HOST_MODEL
// ---------------------------------------------------------------------------
// Cross-lane exchange
// ---------------------------------------------------------------------------
// DPP controls (row = 16 lanes): row_mirror l <-> 15-l, row_half_mirror
// l <-> 7-l, quad_perm [2,3,0,1] l <-> l^2, quad_perm [1,0,3,2] l <-> l^1.
constexpr int kDppMirror16 = 0x140;
constexpr int kDppMirror8 = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Partner of a lane across lane bit MASK (8, 4, 2, 1) uses the mirror/perm
// that flips that bit and keeps all higher bits.
template <int MASK>
__device__ __forceinline__ float dpp_partner(float v) {
  if constexpr (MASK == 8) return dpp_f<kDppMirror16>(v);
  else if constexpr (MASK == 4) return dpp_f<kDppMirror8>(v);
  else if constexpr (MASK == 2) return dpp_f<kDppXor2>(v);
  else return dpp_f<kDppXor1>(v);
}

// Swap step across lane bit 5 (MASK 32) or 4 (MASK 16) on a pair (a, b):
// afterwards a lane with the bit clear holds a + partner's a, a lane with the
// bit set holds b + partner's b.
template <int MASK>
__device__ __forceinline__ float swap_pair_sum(float a, float b) {
  if constexpr (MASK == 32) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// ---------------------------------------------------------------------------
// Transposed team reduction
// ---------------------------------------------------------------------------
// A team of LANES lanes (8, 16, 32 or 64, aligned inside the wave) holds P
// planes of V partial sums per lane. Summing every value over the team would
// cost log2(LANES) exchanges per value; instead each exchange step halves the
// number of values a lane carries: across lane bit b, a lane with b clear
// keeps the even value of each pair and one with b set the odd value, each
// adding its partner's copy of the kept value. After S = min(log2 V,
// log2 LANES) such steps, the remaining steps are plain pairwise sums. Value
// position i of lane l then holds the team total of value index
//   i * 2^S + sum_{k<S} bit_{L-1-k}(l) * 2^k      (L = log2 LANES),
// identical in every lane whose top S bits (within the team) agree. V must be
// a power of two. Every plane is reduced with the same lane mapping.
template <int LANES>
constexpr int log2i() { return LANES <= 1 ? 0 : 1 + log2i<LANES / 2>(); }

// One step across lane bit MASK on the first C values of every plane.
template <int MASK, int P, int V, int C>
__device__ __forceinline__ void reduce_step(float (&v)[P][V], int lane) {
  if constexpr (C > 1) {
    const bool bit = (lane & MASK) != 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int i = 0; i < C / 2; ++i) {
        const float a = v[p][2 * i], b = v[p][2 * i + 1];
        if constexpr (MASK >= 16) {
          v[p][i] = swap_pair_sum<MASK>(a, b);
        } else {
          const float keep = bit ? b : a;
          const float send = bit ? a : b;
          v[p][i] = keep + dpp_partner<MASK>(send);
        }
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if constexpr (MASK >= 16) v[p][0] = swap_pair_sum<MASK>(v[p][0], v[p][0]);
      else v[p][0] = v[p][0] + dpp_partner<MASK>(v[p][0]);
    }
  }
}

template <int MASK, int P, int V, int C>
__device__ __forceinline__ void reduce_from(float (&v)[P][V], int lane) {
  if constexpr (MASK >= 1) {
    reduce_step<MASK, P, V, C>(v, lane);
    reduce_from<MASK / 2, P, V, (C > 1 ? C / 2 : 1)>(v, lane);
  }
}

// Reduces in place; afterwards v[p][0 .. V/2^S) are valid.
template <int LANES, int P, int V>
__device__ __forceinline__ void team_reduce(float (&v)[P][V], int lane) {
  static_assert((V & (V - 1)) == 0, "V must be a power of two");
  reduce_from<LANES / 2, P, V, V>(v, lane);
}

template <int LANES, int V>
struct ReduceMap {
  static constexpr int L = log2i<LANES>();
  static constexpr int S = log2i<V>() < L ? log2i<V>() : L;
  static constexpr int kPerLane = V >> S;       // positions a lane holds
  // index of the value at position i in the lane with in-team id l
  __device__ static int index(int l, int i) {
    int b = 0;
#pragma unroll
    for (int k = 0; k < S; ++k) b |= ((l >> (L - 1 - k)) & 1) << k;
    return (i << S) | b;
  }
  // one representative lane per distinct result
  __device__ static bool representative(int l) { return (l & ((1 << (L - S)) - 1)) == 0; }
};

#endif  // !QMV_HOST_MODEL

}  // namespace qmv
