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
#include "q8.hpp"

namespace qmv {

__global__ void __launch_bounds__(256) quantize_q8_1_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ y, int64_t nb,
                                                            int64_t n, int64_t ldx) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // 256-lane blocks
  const int64_t blk = gid >> 3;          // global q8_1 block (column-major over n)
  const int sub = static_cast<int>(gid & 7);
  const bool valid = blk < n * nb;
  const int64_t bc = valid ? blk : 0;    // no early exit: the group reduces with DPP
  const int64_t j = bc / nb, b = bc - j * nb;
  const u32x4 raw[1] = {ld_x4(reinterpret_cast<const uint8_t*>(x + j * ldx + 32 * b + 4 * sub))};

  float amax = absmax4(raw[0]);
  amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_f<kDppMirror8>(amax));

  const float d = q8_scale(amax);
  int sq = 0;
  uint32_t packed[1];
  q8_quant_block(raw, d, packed, sq);
  sq += __builtin_amdgcn_update_dpp(0, sq, kDppXor1, 0xF, 0xF, false);
  sq += __builtin_amdgcn_update_dpp(0, sq, kDppXor2, 0xF, 0xF, false);
  sq += __builtin_amdgcn_update_dpp(0, sq, kDppMirror8, 0xF, 0xF, false);

  if (!valid) return;
  uint8_t* yb = y + bc * kQ8Bytes;
  *reinterpret_cast<uint32_t*>(yb + 4 + 4 * sub) = packed[0];
  if (sub == 0) *reinterpret_cast<uint32_t*>(yb) = f2h_bits(d) | (f2h_bits(q8_s(d, sq)) << 16);
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
