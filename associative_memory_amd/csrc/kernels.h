// Kernel launchers of libkata (internal C++ interface between the C ABI layer
// and the HIP kernels).  Every launcher assumes its arguments were validated
// by the caller (api.cpp) and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kata {

// phi(x) for `rows` vectors of width d (public sqrt(2) packing).
hipError_t launch_feature_map(const void* x, void* phi, int64_t rows, int d,
                              bool x_bf16, bool phi_bf16, hipStream_t stream);

// One recurrent step for BH independent heads.
hipError_t launch_decode(float* S, float* z, const void* q, const void* k,
                         const void* v, void* out, int64_t BH, int d, int dv,
                         float eps, bool bf16, hipStream_t stream);
// One gated step (S = gamma S + phi(k) v^T, o = phi(q)^T S; no z).
hipError_t launch_decode_gated(float* S, const void* q, const void* k, const void* v,
                               const float* log_gamma, void* out, int64_t BH, int d, int dv,
                               bool bf16, hipStream_t stream);

// Sums over spans of tokens:
//   S_out[(bh*n_spans+sp)*s_stride + f*dv + c] = sum_t w_f k_i k_j v_t[c]
//   z_out[(bh*n_spans+sp)*z_stride + f]        = sum_t w_f k_i k_j
// over tokens t in [sp*span, min(T, (sp+1)*span)) of head bh, with
// w_f = sqrt(2) off the diagonal when `sym`, else 1.  Spans that are the
// last of their head are skipped when `skip_last` (their sum is not needed
// by an exclusive prefix).
struct StateArgs {
  const void* k;
  const void* v;
  float* S_out;
  float* z_out;
  int64_t BH;
  int64_t T;
  int d;
  int dv;
  int64_t span;      // tokens per span
  int64_t n_spans;   // spans per head
  int64_t s_stride;  // floats between consecutive (bh, span) S blocks
  int64_t z_stride;  // floats between consecutive (bh, span) z blocks
  bool bf16;
  bool sym;
  bool skip_last;
  // gated state (one span per head): S <- exp(log_gamma_t) S + phi(k_t) v_t^T
  // token by token, log_gamma [BH*T]; z_out is not written
  const float* log_gamma = nullptr;
};
hipError_t launch_state_valu(const StateArgs& a, hipStream_t stream);

// In-place exclusive prefix over the span axis of ws[BH][n_spans][E].
hipError_t launch_scan_sequential(float* ws, int64_t BH, int64_t n_spans,
                                  int64_t E, hipStream_t stream);
hipError_t launch_scan_associative(float* ws, int64_t BH, int64_t n_spans,
                                   int64_t E, hipStream_t stream);

// Gated read: half the running gate sums per chunk, beta_t / 2 with
// beta_t = log2(e) * sum of log_gamma from the chunk start to t (gb[BH*T]), key factors
// 2^((beta_C - beta_t) / 2) with beta_C the chunk's last beta (gk[BH*T]), and
// chunk totals (ctot[BH][ceil(T/chunk)]); chunk 64 or 128.
hipError_t launch_gate_prep(const float* log_gamma, float* gb, float* gk, float* ctot, int64_t BH,
                            int64_t T, int chunk, hipStream_t stream);
// In-place exclusive affine prefix over ws[BH][n_spans][E]:
// P_0 = 0, P_{j+1} = 2^(sum of span j's chunk totals) P_j + ws[j].
hipError_t launch_scan_affine(float* ws, const float* ctot, int64_t BH, int64_t n_spans,
                              int64_t E, int64_t G, int64_t n_chunks, hipStream_t stream);
// The same affine prefix by reduce-then-scan (segments of the span axis,
// log-depth combine of the segment maps).
hipError_t launch_scan_affine_associative(float* ws, const float* ctot, int64_t BH,
                                          int64_t n_spans, int64_t E, int64_t G,
                                          int64_t n_chunks, hipStream_t stream);

// Chunked readout with carried state, VALU fp32 arithmetic.  Each workgroup
// takes one span of `G` chunks of one head (and a slice of dv columns),
// starts from the exclusive prefix state of that span (or zero when
// prefix == nullptr), and for each chunk reads out then updates the state.
struct OutputArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* prefix;  // [BH][n_spans][D*dv + D] or nullptr
  int64_t BH;
  int64_t T;
  int d;
  int dv;
  int chunk;
  int64_t G;        // chunks per span
  int64_t n_spans;  // spans per head
  float eps;
  bool bf16;
};
hipError_t launch_output_valu(const OutputArgs& a, hipStream_t stream);

// Measurement aid: a loop of independent bf16 16x16x32 matrix-core products,
// `workgroups` workgroups of 4 waves, `iters` rounds of 8 products per wave;
// each thread writes one sum to sink[workgroups * 256].
hipError_t launch_probe_mfma(float* sink, int workgroups, int iters, hipStream_t stream);
int64_t probe_mfma_flops(int workgroups, int iters);

}  // namespace kata
