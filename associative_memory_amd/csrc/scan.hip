// Exclusive prefix over span states (the KATA page, Sec. 4.2 and App. E.1:
// the chunk-state recurrence of Eq. 17 is a vector-space cumulative sum, so
// its prefix can be taken sequentially, depth N, or, by associativity, as a
// parallel scan: segments of the span axis reduced in order and their
// results combined in log-depth rounds).  Both kernels work in place on
// ws[BH][N][E], fp32, and leave P[0] = 0, P[n] = sum_{m<n} A[m] for every
// element.
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

// Associative, reduce-then-scan.  The span axis of every element is cut into
// L segments of M = ceil(N / L) spans.  A thread first reduces its segment
// (the element's spans in order), the L segment results of an element are
// then scanned in LDS by Hillis-Steele in log2 L rounds (the combine is
// associative), and each thread finally walks its segment again from the
// exclusive result of the segments before it.  A workgroup holds EL =
// kThreads / L consecutive elements times L segments, so one load
// instruction of a wave reads runs of EL consecutive floats.  With M at most
// the register batch U the segment stays in registers between the two walks (one read, one
// write per entry).
//
// ADD: the prefix of Eq. 17, P_{n+1} = P_n + A_n.
// !ADD (gated read): P_{n+1} = a_n P_n + A_n with the span decays a_n in
// LDS; a segment reduces to the pair (product of its decays, its walk from
// zero) and pairs compose as (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2).
constexpr int kScanBatch = 16;  // entries a thread keeps in registers

template <int L, bool ADD>
__global__ __launch_bounds__(kThreads) void scan_blocked_kernel(float* __restrict__ ws,
                                                                const float* __restrict__ ctot,
                                                                int64_t N, int64_t E,
                                                                int64_t tiles, int64_t G,
                                                                int64_t n_chunks) {
  constexpr int EL = kThreads / L;
  constexpr int U = kScanBatch;
  extern __shared__ float decay[];  // !ADD only: N span decays
  __shared__ float red[2][L][EL];   // segment results: decay product, sum
  const int64_t bh = blockIdx.x / tiles;
  if (!ADD) {
    for (int64_t j = threadIdx.x; j < N; j += kThreads) {
      float sum = 0.f;
      const int64_t c1 = (j + 1) * G < n_chunks ? (j + 1) * G : n_chunks;
      for (int64_t c = j * G; c < c1; ++c) sum += ctot[bh * n_chunks + c];
      decay[j] = exp2f(sum);
    }
    __syncthreads();
  }
  const int el = threadIdx.x % EL, seg = threadIdx.x / EL;
  const int64_t e = (blockIdx.x - bh * tiles) * EL + el;
  const bool live = e < E;
  // 32-bit offsets inside one head's N x E block (the launcher checks N E < 2^31)
  const int Ei = static_cast<int>(E);
  const int M = static_cast<int>((N + L - 1) / L);
  const int n0 = seg * M;
  const int cnt = static_cast<int>(N) - n0 < M ? static_cast<int>(N) - n0 : M;  // <= 0: empty
  const int last = cnt > 0 ? n0 + cnt - 1 : 0;
  float* base = ws + bh * N * E + (live ? e : 0);
  auto step = [&](float run, int n, float x) {
    return ADD ? run + x : __builtin_fmaf(decay[n], run, x);
  };
  // loads are unconditional (clamped to the segment's last entry) so that a
  // batch issues back to back; out-of-segment values are never used
  auto load_batch = [&](float (&a)[U], int n) {
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = base[(n + u < last ? n + u : last) * Ei];
  };

  float a[U];
  float prod = 1.f, sum = 0.f;
  for (int n = n0; n < n0 + cnt; n += U) {
    load_batch(a, n);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (n + u < n0 + cnt) {
        sum = step(sum, n + u, a[u]);
        if (!ADD) prod *= decay[n + u];
      }
    }
  }

  red[0][seg][el] = prod;
  red[1][seg][el] = sum;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < L; off <<= 1) {
    float pa = 1.f, pb = 0.f;
    if (seg >= off) {
      pa = red[0][seg - off][el];
      pb = red[1][seg - off][el];
    }
    __syncthreads();
    if (seg >= off) {
      // this segment's (inclusive) result applied after the earlier ones
      const float qa = red[0][seg][el], qb = red[1][seg][el];
      red[0][seg][el] = ADD ? 1.f : qa * pa;
      red[1][seg][el] = ADD ? pb + qb : __builtin_fmaf(qa, pb, qb);
    }
    __syncthreads();
  }
  if (!live) return;
  float run = seg > 0 ? red[1][seg - 1][el] : 0.f;  // exclusive result

  // with cnt <= U the batch is still in registers; otherwise read again
  for (int n = n0; n < n0 + cnt; n += U) {
    if (cnt > U) load_batch(a, n);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (n + u < n0 + cnt) {
        base[(n + u) * Ei] = run;
        run = step(run, n + u, a[u]);
      }
    }
  }
}

// Segments per element: enough that a segment fits the register batch (up to
// 16, where a wave still reads runs of 16 consecutive floats).
int scan_segments(int64_t N) {
  int L = 1;
  while (L < 16 && static_cast<int64_t>(L) * kScanBatch < N) L *= 2;
  return L;
}

template <bool ADD>
hipError_t launch_blocked(float* ws, const float* ctot, int64_t BH, int64_t N, int64_t E,
                          int64_t G, int64_t n_chunks, hipStream_t stream) {
  if (!ADD && N > 8192) return hipErrorInvalidValue;  // span decays in LDS
  if (N * E > INT32_MAX) return hipErrorInvalidValue;
  const int L = scan_segments(N);
  const int64_t EL = kThreads / L;
  const int64_t tiles = (E + EL - 1) / EL;
  dim3 grid(static_cast<unsigned>(tiles * BH));
  const size_t lds = ADD ? 0 : N * sizeof(float);
  switch (L) {
#define KATA_SCAN_L(LL)                                                                   \
  case LL:                                                                                \
    scan_blocked_kernel<LL, ADD><<<grid, kThreads, lds, stream>>>(ws, ctot, N, E, tiles, G, \
                                                                  n_chunks);              \
    break;
    KATA_SCAN_L(1)
    KATA_SCAN_L(2)
    KATA_SCAN_L(4)
    KATA_SCAN_L(8)
    KATA_SCAN_L(16)
#undef KATA_SCAN_L
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Gated read (GatedKATA): the state recurrence S_t = gamma_t S_{t-1} +
// phi(k_t) v_t^T makes the prefix over spans affine, P_0 = 0,
// P_{j+1} = a_j P_j + A_j with a_j the product of the gates over span j.
//
// gate_prep_kernel: one wave per chunk of C tokens writes half the running
// gate sums, beta_t / 2 with beta_t = log2(e) sum_{c0 <= r <= t} log gamma_r
// (inclusive, from the chunk start c0; the readout's factors are all square
// roots 2^((beta_t - beta_s) / 2), so the halves save a multiply each), the
// key factors 2^((beta_C - beta_t) / 2) that scale key row t in the chunk's
// state update (beta_C = beta at the chunk's last token), and the chunk total
// beta_C; a lane holds C/64 consecutive tokens.
constexpr float kHalfLog2e = 0.72134752044448170368f;

template <int C>
__global__ __launch_bounds__(kThreads) void gate_prep_kernel(const float* __restrict__ lg,
                                                             float* __restrict__ gb,
                                                             float* __restrict__ gk,
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
    run += (t < T) ? lg[bh * T + t] * kHalfLog2e : 0.f;
    x[i] = run;
  }
  float incl = run;  // inclusive prefix of the lane totals over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const float excl = incl - run;
  const float beta_c = __shfl(excl + x[PER - 1], 63);  // beta_C / 2
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (t0 + i < T) {
      gb[bh * T + t0 + i] = excl + x[i];
      gk[bh * T + t0 + i] = __builtin_amdgcn_exp2f(beta_c - (excl + x[i]));
    }
  }
  if (lane == 63) ctot[bh * n_chunks + c] = 2.f * incl;
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

hipError_t launch_gate_prep(const float* log_gamma, float* gb, float* gk, float* ctot, int64_t BH,
                            int64_t T, int chunk, hipStream_t stream) {
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  const int64_t waves = BH * n_chunks;
  dim3 grid(static_cast<unsigned>((waves + kThreads / 64 - 1) / (kThreads / 64)));
  if (chunk == 64) {
    gate_prep_kernel<64><<<grid, kThreads, 0, stream>>>(log_gamma, gb, gk, ctot, BH, T, n_chunks);
  } else if (chunk == 128) {
    gate_prep_kernel<128><<<grid, kThreads, 0, stream>>>(log_gamma, gb, gk, ctot, BH, T, n_chunks);
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
  return launch_blocked<true>(ws, nullptr, BH, N, E, 1, N, stream);
}

hipError_t launch_scan_affine_associative(float* ws, const float* ctot, int64_t BH, int64_t N,
                                          int64_t E, int64_t G, int64_t n_chunks,
                                          hipStream_t stream) {
  return launch_blocked<false>(ws, ctot, BH, N, E, G, n_chunks, stream);
}

}  // namespace kata
