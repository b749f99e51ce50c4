// Interface of the matrix-core chunked forward (bf16, dv = 64, head dim 16 or
// 32, chunk 64 or 128), the quadratic form, the linear cone features and the
// gated read.  The kernels are in forward_mfma.hip, forward_quadratic.hip and
// forward_linear.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

constexpr int kMfmaValueTiles = 5;  // 4 tiles of 16 value columns + the ones-column tile

// waves per workgroup: the d = 32 state (33 feature tiles) and the KATA-M4
// state at d = 64 (34 tiles) are spread over 8
__host__ __device__ constexpr int mfma_waves(int d) { return d == 16 ? 4 : 8; }

// feature tiles of 16 positions holding the features: d(d+1)/2 for the full
// map at d = 16, 32; 4 x 136 for the KATA-M4 block map at d = 64
__host__ __device__ constexpr int mfma_feature_tiles(int d) { return d == 16 ? 9 : (d == 32 ? 33 : 34); }

// floats of one span state in the workspace: the fp32 accumulator tiles of
// the 4 value tiles, then the denominator column z (16 floats per feature tile)
__host__ __device__ constexpr int64_t mfma_state_floats(int d) {
  return int64_t(mfma_feature_tiles(d)) * (kMfmaValueTiles - 1) * 256 +
         int64_t(mfma_feature_tiles(d)) * 16;
}

struct MfmaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ws;        // [BH][n_spans][mfma_state_floats(d)]
  int64_t BH;
  int64_t T;
  int d;
  int chunk;
  int64_t G;        // chunks per span
  int64_t n_spans;  // spans per head
  // paired spans (d = 16 kernels): with GL > 0 the spans come in pairs of 2G
  // chunks, the even span of a pair GL chunks and the odd one 2G - GL
  int64_t GL = 0;
  float eps;
  const float* gb = nullptr;  // gated read: half the running gate sums per token, log2 units
  const float* gk = nullptr;  // gated read: key factors 2^((beta_C - beta_t) / 2) per token
  float* part = nullptr;      // sliced maps: fp32 partial reads [BH*T][68]
  int fm = 0;                 // sliced maps: 100 + slice (KATA-M1), 200 + slice (KATA-M2)
  // d = 16, ungated: each readout workgroup forms its span's prefix from the
  // head's earlier chunks (no span sums, no prefix, no workspace)
  bool recompute = false;
  // d = 16, ungated: the readout workgroup of span j adds the stored span
  // sums of spans 0 .. j - 1 itself (no prefix launch)
  bool fused = false;
};

struct QuadArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t BH;
  int64_t T;
  int d;
  int g;  // feature blocks (KATA-Mg); 1 = the full rank-one map
  float eps;
};

// bf16, dv = 64, d in {16, 32, 64} split into g blocks of width 16, 32 or 64
inline bool quadratic_supported(bool bf16, int d, int dv, int g) {
  if (!bf16 || dv != 64 || g < 1 || d % g != 0) return false;
  if (d != 16 && d != 32 && d != 64) return false;
  const int m = d / g;
  return m == 16 || m == 32 || m == 64;
}

// the O(T^2) form: one workgroup per (head, 128-query block)
hipError_t launch_forward_quadratic_mfma(const QuadArgs& a, hipStream_t stream);

// ------------------------------------------------------------ linear features
// (D = d = 64, chunk 32, 64 or 128): orthant psi(x) = ReLU(x) + shift,
// Lorentz psi(x) = (y, |y| (1 + s^2)) (normalised reads), identity psi(x) = x
// (first-order read, no denominator)
constexpr int kLinFeatOrthant = 0;
constexpr int kLinFeatLorentz = 1;
constexpr int kLinFeatIdentity = 2;
// floats of one span state: 4 feature tiles x 5 value tiles of accumulator
// tiles (the ones-column tile holds z in its first column); the identity map
// keeps 4 value tiles (4096 floats)
constexpr int64_t kLinStateFloats = int64_t(4) * kMfmaValueTiles * 256;
int64_t linear_state_floats(int feature);

struct LinArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ws;  // [BH][n_spans][linear_state_floats(feature)]
  int64_t BH;
  int64_t T;
  int feature;
  float shift;
  int64_t G;        // chunks per span
  int64_t n_spans;  // spans per head
  float eps;
  int chunk = 64;   // chunk length: 32, 64 or 128
};

inline bool linear_supported(bool bf16, int d, int dv, int chunk) {
  return bf16 && d == 64 && dv == 64 && (chunk == 32 || chunk == 64 || chunk == 128);
}

// span sums psi(K)^T [V | 1] of spans 0 .. n_spans-2 of every head into ws
hipError_t launch_linear_span_state(const LinArgs& a, hipStream_t stream);
// readout of every span from the exclusive prefix in ws
hipError_t launch_linear_readout(const LinArgs& a, hipStream_t stream);

inline bool mfma_supported(bool bf16, int d, int dv, int chunk) {
  return bf16 && (d == 16 || d == 32) && dv == 64 && (chunk == 64 || chunk == 128);
}

// readout workgroups that form their span's prefix themselves (KATA_SCAN_RECOMPUTE)
inline bool recompute_supported(bool bf16, int d, int dv, int chunk) {
  return mfma_supported(bf16, d, dv, chunk) && d == 16;
}

// readout workgroups that add the stored span sums before their span
// (KATA_SCAN_FUSED): the d = 16 readout and the wave-specialised d = 32 one
inline bool fused_supported(bool bf16, int d, int dv, int chunk) {
  return mfma_supported(bf16, d, dv, chunk) && (d == 16 || chunk == 64);
}

// the chunked reads at d = 64: KATA-M4 (g = 4, blocks of 16), KATA-M2 (g = 2,
// two slices of the feature axis) and the full map KATA-M1 (g = 1, four
// slices); bf16, dv = 64, chunk 64
inline bool block_map_supported(bool bf16, int d, int dv, int g, int chunk) {
  return bf16 && d == 64 && (g == 1 || g == 2 || g == 4) && dv == 64 && chunk == 64;
}
constexpr int kPartFloats = 68;  // fp32 partial read per token: 64 values, denominator, padding

// span sums of spans 0 .. n_spans-2 of every head into ws
hipError_t launch_span_state_mfma(const MfmaArgs& a, hipStream_t stream);
// readout of every span, starting from the exclusive prefix in ws
hipError_t launch_readout_mfma(const MfmaArgs& a, hipStream_t stream);

// The gated read (GatedKATA) on the d = 16 and d = 32 paths, chunk 64 or 128:
// span sums and readout with the running gate sums a.gb and key factors a.gk
// (no denominator).
inline bool gated_supported(bool bf16, int d, int dv, int chunk) {
  return bf16 && (d == 16 || d == 32) && dv == 64 && (chunk == 64 || chunk == 128);
}
hipError_t launch_span_state_gated(const MfmaArgs& a, hipStream_t stream);
hipError_t launch_readout_gated(const MfmaArgs& a, hipStream_t stream);

}  // namespace kata
