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
// grid.x enumerates (bh, span, dv tile).  Thread slot m owns feature
// f = tid + m * kThreads with all DVT columns of the tile: per token it reads
// its two key coordinates and the token's DVT values (one broadcast row), so
// the product k_i k_j is formed once per feature and token.  z is summed by
// the dv tile 0 workgroup.
//
// GATED (a.log_gamma != nullptr, one span per head): the GatedKATA state of
// the span, S <- gamma_t S + phi(k_t) v_t^T token by token (the page, App.
// F.4), with gamma_t = exp(log_gamma_t); no z.
template <int DK, bool BF16, bool GATED = false>
__global__ __launch_bounds__(kThreads) void state_valu_kernel(StateArgs a) {
  constexpr int D = feature_dim(DK);
  constexpr int MF = (D + kThreads - 1) / kThreads;  // features per thread
  __shared__ float ks[TT][DK];
  __shared__ alignas(16) float vs[TT][DVT];
  __shared__ float gs[GATED ? TT : 1];

  const int n_tiles = a.dv / DVT;
  int64_t id = blockIdx.x;
  const int tile = static_cast<int>(id % n_tiles);
  id /= n_tiles;
  const int64_t sp = id % a.n_spans;
  const int64_t bh = id / a.n_spans;
  if (a.skip_last && sp == a.n_spans - 1) return;
  const int tid = threadIdx.x;

  int fi[MF], fj[MF];
  float acc[MF][DVT];
  float zacc[MF];
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int f = tid + m * kThreads;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    fi[m] = i;
    fj[m] = j;
    zacc[m] = 0.f;
#pragma unroll
    for (int c = 0; c < DVT; ++c) acc[m][c] = 0.f;
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
      float vr[DVT];
#pragma unroll
      for (int c4 = 0; c4 < DVT / 4; ++c4) {
        const float4 x = reinterpret_cast<const float4*>(vs[r])[c4];
        vr[4 * c4] = x.x;
        vr[4 * c4 + 1] = x.y;
        vr[4 * c4 + 2] = x.z;
        vr[4 * c4 + 3] = x.w;
      }
      const float g = GATED ? gs[r] : 1.f;
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if (m + 1 < MF || tid + m * kThreads < D) {
          const float p = ks[r][fi[m]] * ks[r][fj[m]];
#pragma unroll
          for (int c = 0; c < DVT; ++c) {
            if constexpr (GATED) {
              acc[m][c] = __builtin_fmaf(acc[m][c], g, p * vr[c]);
            } else {
              acc[m][c] = __builtin_fmaf(p, vr[c], acc[m][c]);
            }
          }
          zacc[m] += p;
        }
      }
    }
    __syncthreads();
  }

  float* So = a.S_out + (bh * a.n_spans + sp) * a.s_stride;
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int f = tid + m * kThreads;
    if (f < D) {
      const float w = (a.sym && fi[m] != fj[m]) ? kSqrt2 : 1.0f;
#pragma unroll
      for (int c = 0; c < DVT; ++c) So[static_cast<int64_t>(f) * a.dv + tile * DVT + c] = w * acc[m][c];
    }
  }
  if (!GATED && tile == 0) {
    float* zo = a.z_out + (bh * a.n_spans + sp) * a.z_stride;
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int f = tid + m * kThreads;
      if (f < D) {
        const float w = (a.sym && fi[m] != fj[m]) ? kSqrt2 : 1.0f;
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
//
// The TPQ threads of a query row split its work and add their partial reads
// by a butterfly over their lanes (each ends with the same sums): thread cg
// takes the packed feature rows p and DK - 1 - p (DK + 1 features together)
// for p = cg, cg + TPQ, ... in the inter-chunk term, and the keys s = cg,
// cg + TPQ, ... of the chunk in the intra-chunk term; it stores value columns
// cg * CPT .. + CPT - 1.  The state update gives each thread whole feature
// rows (all DVT columns), so k_i k_j is formed once per feature and token.
template <int DK, int C, bool BF16>
__global__ __launch_bounds__(kThreads) void output_valu_kernel(OutputArgs a) {
  constexpr int D = feature_dim(DK);
  constexpr int TPQ = kThreads / C;   // threads per query row
  constexpr int CPT = DVT / TPQ;      // value columns each thread stores
  constexpr int KP = DK + 4;          // q / k row stride (16-byte rows)
  constexpr int MF = (D + kThreads - 1) / kThreads;  // feature rows per thread in the update
  static_assert(TPQ * C == kThreads && CPT * TPQ == DVT, "bad tiling");
  static_assert((DK / 2) % TPQ == 0, "row pairs split evenly over a query's threads");

  __shared__ alignas(16) float Ss[D][DVT];
  __shared__ float zs[D];
  __shared__ alignas(16) float qs[C][KP];
  __shared__ alignas(16) float ks[C][KP];
  __shared__ alignas(16) float vs[C][DVT];

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
    Ss[f][c] = P ? P[static_cast<int64_t>(f) * a.dv + tile * DVT + c] : 0.f;
  }
  for (int f = tid; f < D; f += kThreads) zs[f] = P ? P[static_cast<int64_t>(D) * a.dv + f] : 0.f;

  int fi[MF], fj[MF];
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int f = tid + m * kThreads;
    int i = 0, j = 0;
    if (f < D) pair_of(f, DK, i, j);
    fi[m] = i;
    fj[m] = j;
  }

  const int tq = tid / TPQ;          // query row within the chunk
  const int cg = tid - tq * TPQ;     // thread within the row's group
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

    float num[DVT];
#pragma unroll
    for (int c = 0; c < DVT; ++c) num[c] = 0.f;
    float den = 0.f;
    // inter-chunk term: phi_q(q_t) . S and phi_q(q_t) . z over this thread's
    // feature rows
    for (int pp = cg; pp < DK / 2; pp += TPQ) {
      const int i0 = pp, i1 = DK - 1 - pp;
      const float qa = qs[tq][i0], qb = qs[tq][i1];
      const int f0 = i0 * DK - i0 * (i0 - 1) / 2;  // first packed feature of row i0
      const int f1 = i1 * DK - i1 * (i1 - 1) / 2;
      for (int n = 0; n <= DK; ++n) {
        const bool row0 = n < DK - i0;
        const int j = row0 ? i0 + n : n - 1;
        const int f = row0 ? f0 + n : f1 + (n - (DK - i0));
        const bool diag = j == (row0 ? i0 : i1);
        const float pf = (diag ? 1.0f : 2.0f) * (row0 ? qa : qb) * qs[tq][j];
#pragma unroll
        for (int c4 = 0; c4 < DVT / 4; ++c4) {
          const float4 x = reinterpret_cast<const float4*>(Ss[f])[c4];
          num[4 * c4] = __builtin_fmaf(pf, x.x, num[4 * c4]);
          num[4 * c4 + 1] = __builtin_fmaf(pf, x.y, num[4 * c4 + 1]);
          num[4 * c4 + 2] = __builtin_fmaf(pf, x.z, num[4 * c4 + 2]);
          num[4 * c4 + 3] = __builtin_fmaf(pf, x.w, num[4 * c4 + 3]);
        }
        den = __builtin_fmaf(pf, zs[f], den);
      }
    }
    // intra-chunk term: (q_t . k_s)^2 for this thread's keys s <= t
    float xq[DK];
#pragma unroll
    for (int i4 = 0; i4 < DK / 4; ++i4) {
      const float4 x = reinterpret_cast<const float4*>(qs[tq])[i4];
      xq[4 * i4] = x.x;
      xq[4 * i4 + 1] = x.y;
      xq[4 * i4 + 2] = x.z;
      xq[4 * i4 + 3] = x.w;
    }
    for (int s = cg; s <= tq; s += TPQ) {
      float dot = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < DK / 4; ++i4) {
        const float4 x = reinterpret_cast<const float4*>(ks[s])[i4];
        dot = __builtin_fmaf(xq[4 * i4], x.x, dot);
        dot = __builtin_fmaf(xq[4 * i4 + 1], x.y, dot);
        dot = __builtin_fmaf(xq[4 * i4 + 2], x.z, dot);
        dot = __builtin_fmaf(xq[4 * i4 + 3], x.w, dot);
      }
      const float sc = dot * dot;
#pragma unroll
      for (int c4 = 0; c4 < DVT / 4; ++c4) {
        const float4 x = reinterpret_cast<const float4*>(vs[s])[c4];
        num[4 * c4] = __builtin_fmaf(sc, x.x, num[4 * c4]);
        num[4 * c4 + 1] = __builtin_fmaf(sc, x.y, num[4 * c4 + 1]);
        num[4 * c4 + 2] = __builtin_fmaf(sc, x.z, num[4 * c4 + 2]);
        num[4 * c4 + 3] = __builtin_fmaf(sc, x.w, num[4 * c4 + 3]);
      }
      den += sc;
    }
    // the row's TPQ partial reads, added over lanes tq * TPQ .. + TPQ - 1
#pragma unroll
    for (int off = 1; off < TPQ; off <<= 1) {
#pragma unroll
      for (int c = 0; c < DVT; ++c) num[c] += __shfl_xor(num[c], off);
      den += __shfl_xor(den, off);
    }
    const int64_t t = c0 + tq;
    if (t < a.T) {
      const float inv = 1.0f / (den + a.eps);
      const int64_t o = (tok0 + t) * a.dv + tile * DVT;
#pragma unroll
      for (int c = 0; c < DVT; ++c) {
        if (c / CPT == cg) store_elem<BF16>(a.out, o + c, num[c] * inv);
      }
    }

    if (g + 1 < a.G) {
      __syncthreads();  // all readouts of this chunk done before S changes
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        const int f = tid + m * kThreads;
        if (m + 1 < MF || f < D) {
          float su[DVT];
#pragma unroll
          for (int c = 0; c < DVT; ++c) su[c] = 0.f;
          float sz = 0.f;
          for (int r = 0; r < C; ++r) {
            const float p = ks[r][fi[m]] * ks[r][fj[m]];
#pragma unroll
            for (int c4 = 0; c4 < DVT / 4; ++c4) {
              const float4 x = reinterpret_cast<const float4*>(vs[r])[c4];
              su[4 * c4] = __builtin_fmaf(p, x.x, su[4 * c4]);
              su[4 * c4 + 1] = __builtin_fmaf(p, x.y, su[4 * c4 + 1]);
              su[4 * c4 + 2] = __builtin_fmaf(p, x.z, su[4 * c4 + 2]);
              su[4 * c4 + 3] = __builtin_fmaf(p, x.w, su[4 * c4 + 3]);
            }
            sz += p;
          }
#pragma unroll
          for (int c = 0; c < DVT; ++c) Ss[f][c] += su[c];
          zs[f] += sz;
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
