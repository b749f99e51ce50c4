// Internal helpers shared by the libkata kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

constexpr int kThreads = 256;

// fp32 nearest to sqrt(2): the off-diagonal weight of the public packing
// (phi(x)_(i,j) = sqrt(2) x_i x_j for i != j, so phi(q).phi(k) = (q.k)^2,
// the KATA page, Sec. 3.1).
constexpr float kSqrt2 = 1.41421356237309504880f;

__host__ __device__ constexpr int feature_dim(int d) { return d * (d + 1) / 2; }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float x) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
  } else {
    static_cast<float*>(p)[i] = x;
  }
}

// (i, j), i <= j, of packed coordinate f of a d x d upper triangle (row-major).
__host__ __device__ inline void pair_of(int f, int d, int& i, int& j) {
  int row = 0;
  int rem = f;
  while (rem >= d - row) {
    rem -= d - row;
    ++row;
  }
  i = row;
  j = row + rem;
}

}  // namespace kata
