// probe.hip - streaming-read probe: the HBM read ceiling the mat-vec
// kernels are measured against.
//
// Reads a buffer with 16-byte coalesced loads and nothing else: each
// 256-lane workgroup takes one contiguous 8 KiB chunk (two loads per lane in
// flight), the launch shape that read a 33 MB matrix fastest among the shapes
// tried (workgroups of 256 to 1024 lanes, 1 to 16 loads per lane, 256 to
// 8064 workgroups). The loaded words are folded into one value per lane that
// is stored only if it equals a fixed constant, so the loads cannot be
// dropped and (practically) nothing is written.
#include "launch.hpp"

namespace qmv {

constexpr int kProbeLanes = 256;
constexpr int64_t kProbeChunk = 8192;

__global__ void __launch_bounds__(kProbeLanes) read_probe_kernel(const uint8_t* __restrict__ src, int64_t bytes,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeChunk;
  const int64_t p0 = base + 16 * threadIdx.x, p1 = p0 + 16 * kProbeLanes;
  u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
  if (p0 + 16 <= bytes) a = ld_a16_x4(src + p0);
  if (p1 + 16 <= bytes) b = ld_a16_x4(src + p1);
  const uint32_t v = a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  if (v == 0x9E3779B9u) sink[0] = v;
}

int launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t grid = (bytes + kProbeChunk - 1) / kProbeChunk;
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(kProbeLanes), 0, st, src, bytes,
                     sink);
  return check_launch();
}

}  // namespace qmv
