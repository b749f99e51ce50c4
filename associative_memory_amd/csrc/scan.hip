// Exclusive prefix over span states (the KATA page, Sec. 4.2 and App. E.1:
// the chunk-state recurrence of Eq. 17 is a vector-space cumulative sum, so
// its prefix can be taken sequentially, depth N, or by a parallel scan in
// ceil(log2 N) rounds).  Both kernels work in place on ws[BH][N][E], fp32,
// and leave P[0] = 0, P[n] = sum_{m<n} A[m] for every element.
#include "common.h"
#include "kernels.h"

namespace kata {
namespace {

// Sequential: one thread per (head, element) walks the span axis.  Loads are
// batched eight at a time so the walk is not one dependent load per step.
__global__ __launch_bounds__(kThreads) void scan_seq_kernel(float* __restrict__ ws,
                                                            int64_t N, int64_t E,
                                                            int64_t tiles) {
  const int64_t bh = blockIdx.x / tiles;
  const int64_t e = (blockIdx.x - bh * tiles) * kThreads + threadIdx.x;
  if (e >= E) return;
  float* base = ws + bh * N * E + e;
  float run = 0.f;
  constexpr int U = 8;
  int64_t n = 0;
  for (; n + U <= N; n += U) {
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = base[(n + u) * E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      base[(n + u) * E] = run;
      run += a[u];
    }
  }
  for (; n < N; ++n) {
    const float a = base[n * E];
    base[n * E] = run;
    run += a;
  }
}

// Associative: one workgroup per (head, tile of ET elements) holds the whole
// span axis for its tile in LDS and runs a Hillis-Steele inclusive scan in
// ceil(log2 N) rounds (round r adds the entry 2^r spans back), then shifts by
// one span to make it exclusive.
constexpr int kScanLds = 8192;  // floats of LDS per workgroup

__global__ __launch_bounds__(kThreads) void scan_assoc_kernel(float* __restrict__ ws,
                                                              int64_t N, int64_t E, int ET,
                                                              int64_t tiles) {
  __shared__ float buf[kScanLds];
  const int64_t bh = blockIdx.x / tiles;
  const int64_t e0 = (blockIdx.x - bh * tiles) * ET;
  float* base = ws + bh * N * E;
  const int tid = threadIdx.x;
  const int total = static_cast<int>(N) * ET;
  int et = ET;
  if (e0 + et > E) et = static_cast<int>(E - e0);

  for (int p = tid; p < total; p += kThreads) {
    const int n = p / ET, c = p - n * ET;
    buf[p] = (c < et) ? base[n * E + e0 + c] : 0.f;
  }
  __syncthreads();
  for (int off = 1; off < N; off <<= 1) {
    const int shift = off * ET;
    constexpr int K = kScanLds / kThreads;
    float add[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int p = tid + k * kThreads;
      add[k] = (p < total && p >= shift) ? buf[p - shift] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int p = tid + k * kThreads;
      if (p < total) buf[p] += add[k];
    }
    __syncthreads();
  }
  for (int p = tid; p < total; p += kThreads) {
    const int n = p / ET, c = p - n * ET;
    if (c < et) base[n * E + e0 + c] = (n == 0) ? 0.f : buf[p - ET];
  }
}

}  // namespace

hipError_t launch_scan_sequential(float* ws, int64_t BH, int64_t N, int64_t E,
                                  hipStream_t stream) {
  const int64_t tiles = (E + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(tiles * BH));
  scan_seq_kernel<<<grid, kThreads, 0, stream>>>(ws, N, E, tiles);
  return hipGetLastError();
}

hipError_t launch_scan_associative(float* ws, int64_t BH, int64_t N, int64_t E,
                                   hipStream_t stream) {
  if (N > kScanLds) return hipErrorInvalidValue;
  int ET = 1;
  while (ET < 64 && static_cast<int64_t>(ET) * 2 * N <= kScanLds) ET *= 2;
  const int64_t tiles = (E + ET - 1) / ET;
  dim3 grid(static_cast<unsigned>(tiles * BH));
  scan_assoc_kernel<<<grid, kThreads, 0, stream>>>(ws, N, E, ET, tiles);
  return hipGetLastError();
}

}  // namespace kata
