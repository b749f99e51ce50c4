// Measurement aid, not part of the method: the dense bf16 matrix-core rate of
// the device, measured with a loop of independent 16x16x32 products.  Each
// wave keeps 8 accumulator chains so consecutive products never wait for one
// another; the operands are constants, so the loop touches no memory until
// the sums are written out (which keeps the compiler from dropping it).
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace kata {
namespace {

constexpr int kProbeChains = 8;

__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  // bf16 1/64 (0x3c80) in every element, perturbed per lane so no two lanes
  // hold the same operands
  const uint32_t x = 0x3c803c80u + static_cast<uint32_t>(lane & 7);
  const u32x4 a = {x, x, x, x};
  const u32x4 b = {x ^ 1u, x, x, x ^ 1u};
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = mfma(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_mfma(float* sink, int workgroups, int iters, hipStream_t stream) {
  probe_mfma_kernel<<<dim3(static_cast<unsigned>(workgroups)), 256, 0, stream>>>(sink, iters);
  return hipGetLastError();
}

int64_t probe_mfma_flops(int workgroups, int iters) {
  // 4 waves per workgroup, 2 x 16 x 16 x 32 FLOP per product
  return static_cast<int64_t>(workgroups) * 4 * iters * kProbeChains * 2 * 16 * 16 * 32;
}

}  // namespace kata
