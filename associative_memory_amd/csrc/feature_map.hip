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
constexpr int64_t kMaxBlocks = 8192;

// A workgroup builds its pair table once and then takes groups of
// kRowsPerBlock rows, grid-strided: stage the rows' x in LDS, then write
// their features.
template <bool XB, bool PB>
__global__ __launch_bounds__(kThreads) void feature_map_kernel(
    const void* __restrict__ x, void* __restrict__ phi, int64_t rows, int d) {
  __shared__ float xs[kRowsPerBlock * kMaxD];
  __shared__ uint8_t pi[kMaxF];
  __shared__ uint8_t pj[kMaxF];
  const int D = feature_dim(d);
  const int tid = threadIdx.x;

  for (int f = tid; f < D; f += kThreads) {
    int i, j;
    pair_of(f, d, i, j);
    pi[f] = static_cast<uint8_t>(i);
    pj[f] = static_cast<uint8_t>(j);
  }
  const int64_t groups = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t row0 = grp * kRowsPerBlock;
    const int nr = static_cast<int>(rows - row0 < kRowsPerBlock ? rows - row0 : kRowsPerBlock);
    __syncthreads();  // the previous group's reads of xs are done (and the pair table is in place)
    if (XB && d % 8 == 0) {
      // 16-byte loads of 8 bf16 (rows start 16-byte aligned: d * 2 B is a multiple of 16)
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row0 * d);
      for (int e = tid; e < nr * d / 8; e += kThreads) {
        const uint4 u = src[e];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          xs[8 * e + 2 * h] = bf16_bits_to_f32(static_cast<uint16_t>(w[h] & 0xffffu));
          xs[8 * e + 2 * h + 1] = bf16_bits_to_f32(static_cast<uint16_t>(w[h] >> 16));
        }
      }
    } else {
      for (int e = tid; e < nr * d; e += kThreads) xs[e] = load_elem<XB>(x, row0 * d + e);
    }
    __syncthreads();

    const int64_t base = row0 * D;
    if (D % 8 == 0) {
      // runs of 8 consecutive features of one row per thread, consecutive
      // threads on consecutive runs: one 16-byte store (bf16) or two (fp32)
      const int runs = D / 8;
      for (int e = tid; e < nr * runs; e += kThreads) {
        const int r = e / runs;
        const int f0 = 8 * (e - r * runs);
        float y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = pi[f0 + u], j = pj[f0 + u];
          const float w = (i == j) ? 1.0f : kSqrt2;
          y[u] = w * xs[r * d + i] * xs[r * d + j];
        }
        const int64_t o = base + static_cast<int64_t>(r) * D + f0;
        if constexpr (PB) {
          uint4 pk;
          pk.x = static_cast<uint32_t>(f32_to_bf16_bits(y[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[1])) << 16);
          pk.y = static_cast<uint32_t>(f32_to_bf16_bits(y[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[3])) << 16);
          pk.z = static_cast<uint32_t>(f32_to_bf16_bits(y[4])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[5])) << 16);
          pk.w = static_cast<uint32_t>(f32_to_bf16_bits(y[6])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[7])) << 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(phi) + o) = pk;
        } else {
          float4* dst = reinterpret_cast<float4*>(static_cast<float*>(phi) + o);
          dst[0] = make_float4(y[0], y[1], y[2], y[3]);
          dst[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
      }
    } else {
      for (int e = tid; e < nr * D; e += kThreads) {
        const int r = e / D;
        const int f = e - r * D;
        const int i = pi[f];
        const int j = pj[f];
        const float w = (i == j) ? 1.0f : kSqrt2;
        store_elem<PB>(phi, base + e, w * xs[r * d + i] * xs[r * d + j]);
      }
    }
  }
}

}  // namespace

hipError_t launch_feature_map(const void* x, void* phi, int64_t rows, int d,
                              bool x_bf16, bool phi_bf16, hipStream_t stream) {
  // up to 32 workgroups per CU, each taking one or more row groups
  const int64_t groups = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  dim3 grid(static_cast<unsigned>(groups < kMaxBlocks ? groups : kMaxBlocks));
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
