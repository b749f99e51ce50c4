// Launch planning for the chunked forward.
//
// The forward runs as three stages (the KATA page, App. E.1 three-kernel
// pipeline): span states -> exclusive prefix over spans -> chunked readout.
// A span is G consecutive chunks.  With G = 1 the prefix runs over every
// chunk exactly as on the page; with G > 1 the readout workgroup carries the
// state across its G chunks itself (read out, then add phi(K_c)^T V_c), so the
// prefix is taken over far fewer, larger sums and the fp32 state traffic
// through HBM shrinks by G.  The result is the same exclusive prefix over
// chunks, summed in a different order.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kata.h"

namespace kata {

enum class Path { Valu = 0, Mfma = 1 };

struct ForwardPlan {
  int64_t BH = 0;
  int64_t T = 0;
  int d = 0;
  int dv = 0;
  int chunk = 0;
  int D = 0;
  bool bf16 = false;
  kata_scan_t scan = KATA_SCAN_SEQUENTIAL;  // resolved: SEQUENTIAL, ASSOCIATIVE or RECOMPUTE
  Path path = Path::Valu;
  int64_t n_chunks = 0;  // ceil(T / chunk)
  int64_t G = 1;         // chunks per span
  int64_t GL = 0;        // paired spans: chunks of each even span (0: all spans G chunks)
  int64_t n_spans = 1;   // spans per head
  int64_t E = 0;         // floats per state pair: D*dv + D
  int64_t wg_state = 0;  // workgroups of the span-state kernel (0 if not run)
  int64_t wg_output = 0; // workgroups of the readout kernel
  size_t ws_bytes = 0;
  // sliced feature maps (KATA-M1 / KATA-M2 at d = 64): slices, id of slice 0,
  // and the byte offset of the fp32 partial reads in the workspace
  int nsl = 1;
  int fm_base = 0;
  size_t part_off = 0;
};

// g > 1: the KATA-Mg block map with g blocks (the matrix-core path supports
// g = 4 at d = 64); g = 1: the full rank-one map
ForwardPlan plan_forward(int B, int H, int64_t T, int d, int dv, int chunk,
                         kata_dtype_t dtype, kata_scan_t scan, int g = 1);

void describe_plan(const ForwardPlan& p, char* buf, size_t len);

hipError_t run_forward(const ForwardPlan& p, const void* q, const void* k, const void* v,
                       void* out, float eps, float* ws, const kata_stage_events_t* events,
                       hipStream_t stream);

}  // namespace kata
