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

// Gated read (GatedKATA): the state recurrence S_t = gamma_t S_{t-1} +
// phi(k_t) v_t^T makes the prefix over spans affine, P_0 = 0,
// P_{j+1} = a_j P_j + A_j with a_j the product of the gates over span j.
//
// gate_prep_kernel: one wave per chunk of C tokens writes the running gate
// sums beta_t = log2(e) sum_{c0 <= r <= t} log gamma_r (inclusive, from the
// chunk start c0) and the chunk total; a lane holds C/64 consecutive tokens.
constexpr float kLog2e = 1.44269504088896340736f;

template <int C>
__global__ __launch_bounds__(kThreads) void gate_prep_kernel(const float* __restrict__ lg,
                                                             float* __restrict__ gb,
                                                             float* __restrict__ ctot, int64_t BH,
                                                             int64_t T, int64_t n_chunks) {
  constexpr int PER = C / 64;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (wid >= BH * n_chunks) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int64_t bh = wid / n_chunks, c = wid - bh * n_chunks;
  const int64_t t0 = c * C + lane * PER;
  float x[PER];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t t = t0 + i;
    run += (t < T) ? lg[bh * T + t] * kLog2e : 0.f;
    x[i] = run;
  }
  float incl = run;  // inclusive prefix of the lane totals over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const float excl = incl - run;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (t0 + i < T) gb[bh * T + t0 + i] = excl + x[i];
  }
  if (lane == 63) ctot[bh * n_chunks + c] = incl;
}

// Sequential affine prefix in place over ws[BH][N][E]: one thread per (head,
// element), the span decays a_j = 2^(sum of the chunk totals of span j) in LDS.
__global__ __launch_bounds__(kThreads) void scan_affine_kernel(float* __restrict__ ws,
                                                               const float* __restrict__ ctot,
                                                               int64_t N, int64_t E, int64_t tiles,
                                                               int64_t G, int64_t n_chunks) {
  extern __shared__ float decay[];
  const int64_t bh = blockIdx.x / tiles;
  for (int64_t j = threadIdx.x; j < N; j += kThreads) {
    float sum = 0.f;
    const int64_t c1 = (j + 1) * G < n_chunks ? (j + 1) * G : n_chunks;
    for (int64_t c = j * G; c < c1; ++c) sum += ctot[bh * n_chunks + c];
    decay[j] = exp2f(sum);
  }
  __syncthreads();
  const int64_t e = (blockIdx.x - bh * tiles) * kThreads + threadIdx.x;
  if (e >= E) return;
  float* base = ws + bh * N * E + e;
  float run = 0.f;
  // loads batched eight at a time, as in the additive walk
  constexpr int U = 8;
  int64_t n = 0;
  for (; n + U <= N; n += U) {
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = base[(n + u) * E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      base[(n + u) * E] = run;
      run = __builtin_fmaf(decay[n + u], run, a[u]);
    }
  }
  for (; n < N; ++n) {
    const float a = base[n * E];
    base[n * E] = run;
    run = __builtin_fmaf(decay[n], run, a);
  }
}

}  // namespace

hipError_t launch_gate_prep(const float* log_gamma, float* gb, float* ctot, int64_t BH, int64_t T,
                            int chunk, hipStream_t stream) {
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  const int64_t waves = BH * n_chunks;
  dim3 grid(static_cast<unsigned>((waves + kThreads / 64 - 1) / (kThreads / 64)));
  if (chunk == 64) {
    gate_prep_kernel<64><<<grid, kThreads, 0, stream>>>(log_gamma, gb, ctot, BH, T, n_chunks);
  } else if (chunk == 128) {
    gate_prep_kernel<128><<<grid, kThreads, 0, stream>>>(log_gamma, gb, ctot, BH, T, n_chunks);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_scan_affine(float* ws, const float* ctot, int64_t BH, int64_t N, int64_t E,
                              int64_t G, int64_t n_chunks, hipStream_t stream) {
  if (N > 8192) return hipErrorInvalidValue;
  const int64_t tiles = (E + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(tiles * BH));
  scan_affine_kernel<<<grid, kThreads, N * sizeof(float), stream>>>(ws, ctot, N, E, tiles, G, n_chunks);
  return hipGetLastError();
}

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
