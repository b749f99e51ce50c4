// Standalone feature map phi(x) (the KATA page, Sec. 3.1 rank-one lift,
// packed to the d(d+1)/2 upper triangle with sqrt(2) off the diagonal).
// The chunked forward never writes phi to HBM; this kernel serves callers
// that want the features themselves.
#include "common.h"
#include "kernels.h"

namespace kata {
namespace {

constexpr int kRowsPerBlock = 32;
constexpr int kMaxD = 64;
constexpr int kMaxF = kMaxD * (kMaxD + 1) / 2;

template <bool XB, bool PB>
__global__ __launch_bounds__(kThreads) void feature_map_kernel(
    const void* __restrict__ x, void* __restrict__ phi, int64_t rows, int d) {
  __shared__ float xs[kRowsPerBlock * kMaxD];
  __shared__ uint8_t pi[kMaxF];
  __shared__ uint8_t pj[kMaxF];
  const int D = feature_dim(d);
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock;
  const int nr = static_cast<int>(rows - row0 < kRowsPerBlock ? rows - row0 : kRowsPerBlock);

  for (int f = tid; f < D; f += kThreads) {
    int i, j;
    pair_of(f, d, i, j);
    pi[f] = static_cast<uint8_t>(i);
    pj[f] = static_cast<uint8_t>(j);
  }
  for (int e = tid; e < nr * d; e += kThreads) {
    xs[e] = load_elem<XB>(x, row0 * d + e);
  }
  __syncthreads();

  const int64_t base = row0 * D;
  for (int e = tid; e < nr * D; e += kThreads) {
    const int r = e / D;
    const int f = e - r * D;
    const int i = pi[f];
    const int j = pj[f];
    const float w = (i == j) ? 1.0f : kSqrt2;
    store_elem<PB>(phi, base + e, w * xs[r * d + i] * xs[r * d + j]);
  }
}

}  // namespace

hipError_t launch_feature_map(const void* x, void* phi, int64_t rows, int d,
                              bool x_bf16, bool phi_bf16, hipStream_t stream) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  dim3 grid(static_cast<unsigned>(blocks));
  if (x_bf16 && phi_bf16) {
    feature_map_kernel<true, true><<<grid, kThreads, 0, stream>>>(x, phi, rows, d);
  } else if (x_bf16) {
    feature_map_kernel<true, false><<<grid, kThreads, 0, stream>>>(x, phi, rows, d);
  } else if (phi_bf16) {
    feature_map_kernel<false, true><<<grid, kThreads, 0, stream>>>(x, phi, rows, d);
  } else {
    feature_map_kernel<false, false><<<grid, kThreads, 0, stream>>>(x, phi, rows, d);
  }
  return hipGetLastError();
}

}  // namespace kata
