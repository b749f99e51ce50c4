// Recurrent decode step (the KATA page, Sec. 2: additive recurrence
// S_t = S_{t-1} + psi(k_t) v_t^T, Z_t = Z_{t-1} + psi(k_t), normalised read of
// Eq. 2 taken after the update).
//
// One workgroup per head.  The head's state S[D][dv] (fp32, dv contiguous) is
// streamed once: every thread owns a float4 column group and a strided set of
// rows, loads all its rows first (so each lane has all its loads in flight,
// issued before the feature products), adds phi(k)_r v, stores, and
// accumulates phi(q)_r S'_r.  Column sums across
// the row groups and the denominator phi(q).z' are reduced through LDS.
//
// GATED: the GatedKATA step (App. F.4), S_t = gamma_t S_{t-1} + psi(k_t) v_t^T,
// read o_t = psi(q_t)^T S_t with no z and no denominator; gamma_t =
// exp(log_gamma) per head.
#include "common.h"
#include "kernels.h"

namespace kata {
namespace {

template <int DK, int DV, bool BF16, bool GATED = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    float* __restrict__ S, float* __restrict__ z, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v, void* __restrict__ out,
    float eps, const float* __restrict__ log_gamma = nullptr) {
  constexpr int D = feature_dim(DK);
  constexpr int TPR = DV / 4;            // threads per state row (float4 each)
  constexpr int RPP = kThreads / TPR;    // rows per pass
  constexpr int NR = (D + RPP - 1) / RPP;
  constexpr int NZ = (D + kThreads - 1) / kThreads;

  __shared__ float xq[DK];
  __shared__ float xk[DK];
  __shared__ float pq[D];
  __shared__ float pk[D];
  __shared__ float4 red[RPP][TPR];
  __shared__ float dred[kThreads / 64];

  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;

  // q and k go out first, then the state, z and v loads: loads retire in
  // order, so q and k reach LDS without waiting for the state, and the state's
  // latency overlaps the barrier and the feature products.
  float qx = 0.f, kx = 0.f;
  if (tid < DK) {
    qx = load_elem<BF16>(q, bh * DK + tid);
    kx = load_elem<BF16>(k, bh * DK + tid);
  }
  const int r0 = tid / TPR;
  const int c4 = tid - r0 * TPR;
  float4 vv;
  vv.x = load_elem<BF16>(v, bh * DV + c4 * 4 + 0);
  vv.y = load_elem<BF16>(v, bh * DV + c4 * 4 + 1);
  vv.z = load_elem<BF16>(v, bh * DV + c4 * 4 + 2);
  vv.w = load_elem<BF16>(v, bh * DV + c4 * 4 + 3);

  float4* Sh = reinterpret_cast<float4*>(S + bh * static_cast<int64_t>(D) * DV);
  float4 s[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int r = r0 + n * RPP;
    if (r < D) s[n] = Sh[r * TPR + c4];
  }
  float* zh = GATED ? nullptr : z + bh * D;
  float zv[NZ];
  if constexpr (!GATED) {
#pragma unroll
    for (int n = 0; n < NZ; ++n) {
      const int f = tid + n * kThreads;
      if (f < D) zv[n] = zh[f];
    }
  }
  float gamma = 1.f;
  if constexpr (GATED) gamma = __expf(log_gamma[bh]);

  if (tid < DK) {
    xq[tid] = qx;
    xk[tid] = kx;
  }
  __syncthreads();
  for (int f = tid; f < D; f += kThreads) {
    int i, j;
    pair_of(f, DK, i, j);
    const float w = (i == j) ? 1.0f : kSqrt2;
    pq[f] = w * xq[i] * xq[j];
    pk[f] = w * xk[i] * xk[j];
  }
  __syncthreads();  // pq / pk ready

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int r = r0 + n * RPP;
    if (r < D) {
      const float a = pk[r];
      const float b = pq[r];
      float4 t = s[n];
      if constexpr (GATED) {
        t.x *= gamma;
        t.y *= gamma;
        t.z *= gamma;
        t.w *= gamma;
      }
      t.x += a * vv.x;
      t.y += a * vv.y;
      t.z += a * vv.z;
      t.w += a * vv.w;
      Sh[r * TPR + c4] = t;
      acc.x += b * t.x;
      acc.y += b * t.y;
      acc.z += b * t.z;
      acc.w += b * t.w;
    }
  }
  float den = 0.f;
  if constexpr (!GATED) {
#pragma unroll
    for (int n = 0; n < NZ; ++n) {
      const int f = tid + n * kThreads;
      if (f < D) {
        const float t = zv[n] + pk[f];
        zh[f] = t;
        den += pq[f] * t;
      }
    }
  }
  red[r0][c4] = acc;
  if constexpr (!GATED) {
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
    if ((tid & 63) == 0) dred[tid >> 6] = den;
  }
  __syncthreads();

  if (tid < DV) {
    // column tid of the row groups' partial sums (red[r] holds DV floats)
    const float* redf = reinterpret_cast<const float*>(&red[0][0]);
    float tot = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) tot += redf[r * DV + tid];
    if constexpr (GATED) {
      store_elem<BF16>(out, bh * DV + tid, tot);
    } else {
      float dd = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) dd += dred[w];
      store_elem<BF16>(out, bh * DV + tid, tot / (dd + eps));
    }
  }
}

template <int DK, int DV>
hipError_t launch_dv(float* S, float* z, const void* q, const void* k, const void* v,
                     void* out, int64_t BH, float eps, bool bf16, hipStream_t s,
                     const float* log_gamma) {
  dim3 grid(static_cast<unsigned>(BH));
  if (log_gamma != nullptr) {
    if (bf16) {
      decode_kernel<DK, DV, true, true><<<grid, kThreads, 0, s>>>(S, z, q, k, v, out, eps, log_gamma);
    } else {
      decode_kernel<DK, DV, false, true><<<grid, kThreads, 0, s>>>(S, z, q, k, v, out, eps, log_gamma);
    }
  } else if (bf16) {
    decode_kernel<DK, DV, true><<<grid, kThreads, 0, s>>>(S, z, q, k, v, out, eps);
  } else {
    decode_kernel<DK, DV, false><<<grid, kThreads, 0, s>>>(S, z, q, k, v, out, eps);
  }
  return hipGetLastError();
}

template <int DK>
hipError_t launch_d(float* S, float* z, const void* q, const void* k, const void* v,
                    void* out, int64_t BH, int dv, float eps, bool bf16, hipStream_t s,
                    const float* log_gamma) {
  switch (dv) {
    case 16: return launch_dv<DK, 16>(S, z, q, k, v, out, BH, eps, bf16, s, log_gamma);
    case 32: return launch_dv<DK, 32>(S, z, q, k, v, out, BH, eps, bf16, s, log_gamma);
    case 64: return launch_dv<DK, 64>(S, z, q, k, v, out, BH, eps, bf16, s, log_gamma);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(float* S, float* z, const void* q, const void* k,
                         const void* v, void* out, int64_t BH, int d, int dv,
                         float eps, bool bf16, hipStream_t stream) {
  switch (d) {
    case 16: return launch_d<16>(S, z, q, k, v, out, BH, dv, eps, bf16, stream, nullptr);
    case 32: return launch_d<32>(S, z, q, k, v, out, BH, dv, eps, bf16, stream, nullptr);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_gated(float* S, const void* q, const void* k, const void* v,
                               const float* log_gamma, void* out, int64_t BH, int d, int dv,
                               bool bf16, hipStream_t stream) {
  switch (d) {
    case 16: return launch_d<16>(S, nullptr, q, k, v, out, BH, dv, 0.f, bf16, stream, log_gamma);
    case 32: return launch_d<32>(S, nullptr, q, k, v, out, BH, dv, 0.f, bf16, stream, log_gamma);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kata
