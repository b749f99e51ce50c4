// fp32 VALU kernels of the chunked forward (the KATA page, Sec. 4.1
// Eqs. 17-20): span-state sums and the chunked readout with a carried state.
// They serve fp32 inputs (where bf16 matrix-core operands would not meet the
// fp32 accuracy bar) and shapes the matrix-core kernels do not cover, and they
// build decode states.  Workgroups own a slice of DVT value columns so the
// fp32 state slice stays small enough for LDS at d = 32.
#include "common.h"
#include "kernels.h"

namespace kata {
namespace {

constexpr int DVT = 16;  // value columns per workgroup
constexpr int TT = 32;   // tokens per LDS tile in the state kernel

// ---------------------------------------------------------------- span states
//
// grid.x enumerates (bh, span, dv tile).  Thread e-slots own elements
// (f, c) = (e / DVT, e % DVT) of the D x DVT block; z is summed by the dv
// tile 0 workgroup.
//
// GATED (a.log_gamma != nullptr, one span per head): the GatedKATA state of
// the span, S <- gamma_t S + phi(k_t) v_t^T token by token (the page, App.
// F.4), with gamma_t = exp(log_gamma_t); no z.
template <int DK, bool BF16, bool GATED = false>
__global__ __launch_bounds__(kThreads) void state_valu_kernel(StateArgs a) {
  constexpr int D = feature_dim(DK);
  constexpr int M = (D * DVT + kThreads - 1) / kThreads;
  constexpr int MZ = (D + kThreads - 1) / kThreads;
  __shared__ float ks[TT][DK];
  __shared__ float vs[TT][DVT];
  __shared__ float gs[GATED ? TT : 1];

  const int n_tiles = a.dv / DVT;
  int64_t id = blockIdx.x;
  const int tile = static_cast<int>(id % n_tiles);
  id /= n_tiles;
  const int64_t sp = id % a.n_spans;
  const int64_t bh = id / a.n_spans;
  if (a.skip_last && sp == a.n_spans - 1) return;
  const int tid = threadIdx.x;

  int fi[M], fj[M], fc[M];
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = tid + m * kThreads;
    const int f = e / DVT;
    fc[m] = e % DVT;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    fi[m] = i;
    fj[m] = j;
    acc[m] = 0.f;
  }
  int zi[MZ], zj[MZ];
  float zacc[MZ];
#pragma unroll
  for (int m = 0; m < MZ; ++m) {
    const int f = tid + m * kThreads;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    zi[m] = i;
    zj[m] = j;
    zacc[m] = 0.f;
  }

  const int64_t t_begin = sp * a.span;
  int64_t t_end = t_begin + a.span;
  if (t_end > a.T) t_end = a.T;
  const int64_t tok0 = bh * a.T;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
    for (int e = tid; e < TT * DK; e += kThreads) {
      const int r = e / DK, c = e - r * DK;
      const int64_t t = t0 + r;
      ks[r][c] = (t < t_end) ? load_elem<BF16>(a.k, (tok0 + t) * DK + c) : 0.f;
    }
    for (int e = tid; e < TT * DVT; e += kThreads) {
      const int r = e / DVT, c = e - r * DVT;
      const int64_t t = t0 + r;
      vs[r][c] = (t < t_end) ? load_elem<BF16>(a.v, (tok0 + t) * a.dv + tile * DVT + c) : 0.f;
    }
    if (GATED && tid < TT) {
      const int64_t t = t0 + tid;
      gs[tid] = (t < t_end) ? __expf(a.log_gamma[tok0 + t]) : 1.f;  // padding: no decay, no key
    }
    __syncthreads();
    for (int r = 0; r < TT; ++r) {
      if constexpr (GATED) {
        const float g = gs[r];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(acc[m], g, ks[r][fi[m]] * ks[r][fj[m]] * vs[r][fc[m]]);
        continue;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += ks[r][fi[m]] * ks[r][fj[m]] * vs[r][fc[m]];
      if (tile == 0) {
#pragma unroll
        for (int m = 0; m < MZ; ++m) zacc[m] += ks[r][zi[m]] * ks[r][zj[m]];
      }
    }
    __syncthreads();
  }

  float* So = a.S_out + (bh * a.n_spans + sp) * a.s_stride;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = tid + m * kThreads;
    const int f = e / DVT;
    if (f < D) {
      const float w = (a.sym && fi[m] != fj[m]) ? kSqrt2 : 1.0f;
      So[f * a.dv + tile * DVT + fc[m]] = w * acc[m];
    }
  }
  if (!GATED && tile == 0) {
    float* zo = a.z_out + (bh * a.n_spans + sp) * a.z_stride;
#pragma unroll
    for (int m = 0; m < MZ; ++m) {
      const int f = tid + m * kThreads;
      if (f < D) {
        const float w = (a.sym && zi[m] != zj[m]) ? kSqrt2 : 1.0f;
        zo[f] = w * zacc[m];
      }
    }
  }
}

// ---------------------------------------------------------------- readout
//
// grid.x enumerates (bh, span, dv tile).  The state slice S[D][DVT] and z[D]
// live in LDS.  The forward keeps its private state with weight 1 on every
// k_i k_j and puts the off-diagonal factor 2 on the query side, so
// phi_q . phi_k = (q.k)^2 needs no sqrt(2) rounding.
template <int DK, int C, bool BF16>
__global__ __launch_bounds__(kThreads) void output_valu_kernel(OutputArgs a) {
  constexpr int D = feature_dim(DK);
  constexpr int TPQ = kThreads / C;   // threads per query row
  constexpr int CPT = DVT / TPQ;      // value columns per thread
  constexpr int M = (D * DVT + kThreads - 1) / kThreads;
  constexpr int MZ = (D + kThreads - 1) / kThreads;
  static_assert(TPQ * C == kThreads && CPT * TPQ == DVT, "bad tiling");

  __shared__ float Ss[D][DVT];
  __shared__ float zs[D];
  __shared__ float qs[C][DK + 1];
  __shared__ float ks[C][DK + 1];
  __shared__ float vs[C][DVT];

  const int n_tiles = a.dv / DVT;
  int64_t id = blockIdx.x;
  const int tile = static_cast<int>(id % n_tiles);
  id /= n_tiles;
  const int64_t sp = id % a.n_spans;
  const int64_t bh = id / a.n_spans;
  const int tid = threadIdx.x;
  const int64_t E = static_cast<int64_t>(D) * a.dv + D;

  // incoming state: exclusive prefix of this span (zero for the first)
  const float* P = a.prefix ? a.prefix + (bh * a.n_spans + sp) * E : nullptr;
  for (int e = tid; e < D * DVT; e += kThreads) {
    const int f = e / DVT, c = e - f * DVT;
    Ss[f][c] = P ? P[f * a.dv + tile * DVT + c] : 0.f;
  }
  for (int f = tid; f < D; f += kThreads) zs[f] = P ? P[static_cast<int64_t>(D) * a.dv + f] : 0.f;

  int fi[M], fj[M], fc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = tid + m * kThreads;
    const int f = e / DVT;
    fc[m] = e % DVT;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    fi[m] = i;
    fj[m] = j;
  }
  int zi[MZ], zj[MZ];
#pragma unroll
  for (int m = 0; m < MZ; ++m) {
    const int f = tid + m * kThreads;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    zi[m] = i;
    zj[m] = j;
  }

  const int tq = tid / TPQ;          // query row within the chunk
  const int cg = tid - tq * TPQ;     // column group
  const int64_t tok0 = bh * a.T;

  for (int64_t g = 0; g < a.G; ++g) {
    const int64_t c0 = (sp * a.G + g) * C;  // first token of this chunk
    if (c0 >= a.T) break;
    __syncthreads();  // previous chunk's state update done
    for (int e = tid; e < C * DK; e += kThreads) {
      const int r = e / DK, c = e - r * DK;
      const int64_t t = c0 + r;
      const bool in = t < a.T;
      qs[r][c] = in ? load_elem<BF16>(a.q, (tok0 + t) * DK + c) : 0.f;
      ks[r][c] = in ? load_elem<BF16>(a.k, (tok0 + t) * DK + c) : 0.f;
    }
    for (int e = tid; e < C * DVT; e += kThreads) {
      const int r = e / DVT, c = e - r * DVT;
      const int64_t t = c0 + r;
      vs[r][c] = (t < a.T) ? load_elem<BF16>(a.v, (tok0 + t) * a.dv + tile * DVT + c) : 0.f;
    }
    __syncthreads();

    float xq[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) xq[i] = qs[tq][i];
    float num[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) num[cc] = 0.f;
    float den = 0.f;
    // inter-chunk term: phi_q(q_t) . S and phi_q(q_t) . z
    {
      int f = 0;
#pragma unroll
      for (int i = 0; i < DK; ++i) {
#pragma unroll
        for (int j = i; j < DK; ++j, ++f) {
          const float pf = (i == j ? 1.0f : 2.0f) * xq[i] * xq[j];
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc) num[cc] += pf * Ss[f][cg * CPT + cc];
          den += pf * zs[f];
        }
      }
    }
    // intra-chunk term: (q_t . k_s)^2 for s <= t within the chunk
    for (int s = 0; s <= tq; ++s) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < DK; ++i) dot += xq[i] * ks[s][i];
      const float sc = dot * dot;
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) num[cc] += sc * vs[s][cg * CPT + cc];
      den += sc;
    }
    const int64_t t = c0 + tq;
    if (t < a.T) {
      const float inv = 1.0f / (den + a.eps);
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        store_elem<BF16>(a.out, (tok0 + t) * a.dv + tile * DVT + cg * CPT + cc, num[cc] * inv);
      }
    }

    if (g + 1 < a.G) {
      __syncthreads();  // all readouts of this chunk done before S changes
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int e = tid + m * kThreads;
        const int f = e / DVT;
        if (f < D) {
          float s = 0.f;
          for (int r = 0; r < C; ++r) s += ks[r][fi[m]] * ks[r][fj[m]] * vs[r][fc[m]];
          Ss[f][fc[m]] += s;
        }
      }
#pragma unroll
      for (int m = 0; m < MZ; ++m) {
        const int f = tid + m * kThreads;
        if (f < D) {
          float s = 0.f;
          for (int r = 0; r < C; ++r) s += ks[r][zi[m]] * ks[r][zj[m]];
          zs[f] += s;
        }
      }
    }
  }
}

template <int DK>
hipError_t launch_state_d(const StateArgs& a, hipStream_t s) {
  const int64_t blocks = a.BH * a.n_spans * (a.dv / DVT);
  dim3 grid(static_cast<unsigned>(blocks));
  if (a.log_gamma != nullptr) {
    if (a.bf16) {
      state_valu_kernel<DK, true, true><<<grid, kThreads, 0, s>>>(a);
    } else {
      state_valu_kernel<DK, false, true><<<grid, kThreads, 0, s>>>(a);
    }
  } else if (a.bf16) {
    state_valu_kernel<DK, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    state_valu_kernel<DK, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int DK, int C>
hipError_t launch_output_dc(const OutputArgs& a, hipStream_t s) {
  const int64_t blocks = a.BH * a.n_spans * (a.dv / DVT);
  dim3 grid(static_cast<unsigned>(blocks));
  if (a.bf16) {
    output_valu_kernel<DK, C, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    output_valu_kernel<DK, C, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int DK>
hipError_t launch_output_d(const OutputArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 32: return launch_output_dc<DK, 32>(a, s);
    case 64: return launch_output_dc<DK, 64>(a, s);
    case 128: return launch_output_dc<DK, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_valu(const StateArgs& a, hipStream_t stream) {
  if (a.dv % DVT != 0) return hipErrorInvalidValue;
  switch (a.d) {
    case 16: return launch_state_d<16>(a, stream);
    case 32: return launch_state_d<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_output_valu(const OutputArgs& a, hipStream_t stream) {
  if (a.dv % DVT != 0) return hipErrorInvalidValue;
  switch (a.d) {
    case 16: return launch_output_d<16>(a, stream);
    case 32: return launch_output_d<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kata
