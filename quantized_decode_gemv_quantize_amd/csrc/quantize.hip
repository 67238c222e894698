// quantize.hip - fp32 activation -> q8_1 blocks on gfx950.
//
// [MMVQ §激活的量化] = page "llama.cpp 源码完全拆解(十四):mul_mat_vec_q——解码时一条
// 量化权重如何被 dp4a 逐块点积", section 激活的量化.
//
// Per block of 32 values: amax, d = amax/127 (fp32, IEEE division),
// q = roundf(x/d) (0 when d == 0), s = d * sum(q) formed in fp32 from the
// exact integer sum; d and s are stored as fp16 (round to nearest even).
// Eight lanes share a block (4 values each, one 16-byte load): amax and the
// code sum are reduced over the 8 lanes with DPP, each lane writes its four
// codes as one dword and the first lane of the group writes {d, s}.
#include "launch.hpp"

namespace qmv {

__device__ __forceinline__ uint32_t f2h_bits(float v) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v)));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__global__ void __launch_bounds__(256) quantize_q8_1_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ y, int64_t nb,
                                                            int64_t n, int64_t ldx) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;          // global q8_1 block (column-major over n)
  const int sub = static_cast<int>(gid & 7);
  const bool valid = blk < n * nb;
  const int64_t bc = valid ? blk : 0;    // no early exit: the group reduces with DPP
  const int64_t j = bc / nb, b = bc - j * nb;
  const u32x4 raw = ld_x4(reinterpret_cast<const uint8_t*>(x + j * ldx + 32 * b + 4 * sub));
  const float v0 = __uint_as_float(raw.x), v1 = __uint_as_float(raw.y);
  const float v2 = __uint_as_float(raw.z), v3 = __uint_as_float(raw.w);

  float amax = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
  amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_f<kDppMirror8>(amax));

  const float d = amax / 127.0f;
  const bool zero = d == 0.0f;
  const int q0 = zero ? 0 : static_cast<int>(roundf(v0 / d));
  const int q1 = zero ? 0 : static_cast<int>(roundf(v1 / d));
  const int q2 = zero ? 0 : static_cast<int>(roundf(v2 / d));
  const int q3 = zero ? 0 : static_cast<int>(roundf(v3 / d));
  const uint32_t packed = (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
                          ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | (static_cast<uint32_t>(q3) << 24);
  int sq = q0 + q1 + q2 + q3;
  sq += dpp_i<kDppXor1>(sq);
  sq += dpp_i<kDppXor2>(sq);
  sq += dpp_i<kDppMirror8>(sq);

  if (!valid) return;
  uint8_t* yb = y + bc * kQ8Bytes;
  *reinterpret_cast<uint32_t*>(yb + 4 + 4 * sub) = packed;
  if (sub == 0) {
    // s is the fp32 product d*sum(q), then rounded to fp16. The empty asm
    // pins the fp32 result in a register: without it the multiply and the
    // f16 conversion fuse into one v_fma_mixlo_f16, which rounds once.
    float s = d * static_cast<float>(sq);
    asm volatile("" : "+v"(s));
    *reinterpret_cast<uint32_t*>(yb) = f2h_bits(d) | (f2h_bits(s) << 16);
  }
}

int launch_quantize_q8_1(const float* x, uint8_t* y, int64_t K, int64_t n, int64_t ldx, hipStream_t st) {
  const int64_t nb = K / 32;
  const int64_t threads = n * nb * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, x, y, nb,
                     n, ldx);
  return check_launch();
}

}  // namespace qmv
