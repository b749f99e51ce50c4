// Interface of the matrix-core chunked forward (d = 16, dv = 64, bf16,
// chunk 64 or 128).  See forward_mfma.hip for the kernel design.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

constexpr int kMfmaValueTiles = 5;    // 4 tiles of 16 value columns + the ones-column tile
constexpr int kMfmaFeatureTiles = 9;  // feature tiles of 16 holding the 136 features
// floats of one span state in the workspace: the fp32 accumulator tiles of
// the 4 value tiles, then the denominator column z (16 floats per feature tile)
constexpr int64_t kMfmaStateFloats = int64_t(kMfmaFeatureTiles) * (kMfmaValueTiles - 1) * 256 +
                                     int64_t(kMfmaFeatureTiles) * 16;

struct MfmaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ws;        // [BH][n_spans][kMfmaStateFloats]
  int64_t BH;
  int64_t T;
  int chunk;
  int64_t G;        // chunks per span
  int64_t n_spans;  // spans per head
  float eps;
};

inline bool mfma_supported(bool bf16, int d, int dv, int chunk) {
  return bf16 && d == 16 && dv == 64 && (chunk == 64 || chunk == 128);
}

// span sums of spans 0 .. n_spans-2 of every head into ws
hipError_t launch_span_state_mfma(const MfmaArgs& a, hipStream_t stream);
// readout of every span, starting from the exclusive prefix in ws
hipError_t launch_readout_mfma(const MfmaArgs& a, hipStream_t stream);

}  // namespace kata
