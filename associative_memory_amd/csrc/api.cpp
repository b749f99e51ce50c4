// C ABI of libkata: argument validation, launch planning, workspace sizing
// and status codes.  Declarations and the contract live in include/kata.h.
#include "kata.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "plan.h"
#include "plan_mfma.h"

namespace {

using kata::ForwardPlan;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t elem_size(kata_dtype_t t) { return t == KATA_BF16 ? 2 : 4; }

bool dtype_ok(kata_dtype_t t) { return t == KATA_F32 || t == KATA_BF16; }
bool head_dim_ok(int d) { return d == 16 || d == 32; }
bool value_dim_ok(int dv) { return dv == 16 || dv == 32 || dv == 64; }
bool chunk_ok(int c) { return c == 32 || c == 64 || c == 128; }

kata_status_t from_hip(hipError_t e) { return e == hipSuccess ? KATA_OK : KATA_ERR_DEVICE; }

// Shape/value checks shared by the forward, its workspace query and its plan.
kata_status_t check_forward_shape(int B, int H, int64_t T, int d, int dv, int chunk,
                                  kata_dtype_t dtype, kata_scan_t scan) {
  if (B <= 0 || H <= 0 || T <= 0) return KATA_ERR_INVALID_VALUE;
  if (scan != KATA_SCAN_AUTO && scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE &&
      scan != KATA_SCAN_RECOMPUTE && scan != KATA_SCAN_FUSED)
    return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!head_dim_ok(d) || !value_dim_ok(dv) || !chunk_ok(chunk)) return KATA_ERR_UNSUPPORTED;
  if (scan == KATA_SCAN_RECOMPUTE && !kata::recompute_supported(dtype == KATA_BF16, d, dv, chunk))
    return KATA_ERR_UNSUPPORTED;
  if (scan == KATA_SCAN_FUSED && !kata::fused_supported(dtype == KATA_BF16, d, dv, chunk))
    return KATA_ERR_UNSUPPORTED;
  // every element index must fit comfortably in int64 and every grid in 2^31
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

// Every check of kata_forward_chunked except those of the workspace.
kata_status_t check_forward_args(const void* q, const void* k, const void* v, const void* out, int B,
                                 int H, int64_t T, int d, int dv, int chunk, float eps,
                                 kata_dtype_t dtype, kata_scan_t scan) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return KATA_ERR_INVALID_VALUE;
  const kata_status_t st = check_forward_shape(B, H, T, d, dv, chunk, dtype, scan);
  if (st != KATA_OK) return st;
  if (!std::isfinite(eps) || eps < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KATA_ERR_INVALID_VALUE;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  if (overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes))
    return KATA_ERR_INVALID_VALUE;
  return KATA_OK;
}

// Span plan of the linear-feature forward: about 512 readout workgroups.
struct LinPlan {
  int64_t n_chunks, G, n_spans;
  size_t ws_bytes;
};

// The workspace is sized for the largest span state (the normalised maps'
// [S | z]); the identity map uses the first 4096 floats of each.
LinPlan plan_linear(int64_t BH, int64_t T, int chunk) {
  LinPlan p;
  p.n_chunks = (T + chunk - 1) / chunk;
  const int64_t spans = (512 + BH - 1) / BH;
  p.G = (p.n_chunks + spans - 1) / spans;
  p.n_spans = (p.n_chunks + p.G - 1) / p.G;
  p.ws_bytes = p.n_spans > 1 ? static_cast<size_t>(BH * p.n_spans * kata::kLinStateFloats) * sizeof(float) : 0;
  return p;
}

kata_status_t check_linear_shape(int B, int H, int64_t T, int d, int dv, int chunk,
                                 kata_feature_t feature, kata_dtype_t dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0 || chunk <= 0) return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (feature != KATA_FEATURE_ORTHANT && feature != KATA_FEATURE_LORENTZ && feature != KATA_FEATURE_IDENTITY)
    return KATA_ERR_INVALID_VALUE;
  if (!kata::linear_supported(dtype == KATA_BF16, d, dv, chunk)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

// Workspace of the gated read: span states (when there are several spans),
// then half the running gate sums [BH*T], the key factors [BH*T] and the chunk
// totals [BH][n_chunks], each 256-byte aligned.
struct GatedLayout {
  ForwardPlan p;
  size_t gb_off = 0, gk_off = 0, ctot_off = 0, bytes = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

GatedLayout plan_gated(int B, int H, int64_t T, int d, int dv, int chunk) {
  GatedLayout l;
  l.p = kata::plan_forward(B, H, T, d, dv, chunk, KATA_BF16, KATA_SCAN_SEQUENTIAL);
  l.gb_off = align256(l.p.ws_bytes);
  l.gk_off = align256(l.gb_off + static_cast<size_t>(l.p.BH * T) * sizeof(float));
  l.ctot_off = align256(l.gk_off + static_cast<size_t>(l.p.BH * T) * sizeof(float));
  l.bytes = l.ctot_off + static_cast<size_t>(l.p.BH * l.p.n_chunks) * sizeof(float);
  return l;
}

kata_status_t check_gated_shape(int B, int H, int64_t T, int d, int dv, int chunk, kata_dtype_t dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0 || chunk <= 0) return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!kata::gated_supported(dtype == KATA_BF16, d, dv, chunk)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH) return KATA_ERR_UNSUPPORTED;
  return KATA_OK;
}

// ------------------------------------------------------------ static scratch
//
// The workspace of kata_forward_chunked_noalloc: one array per device, part of
// the library's code object (each device the library runs on holds it until
// the process ends).  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[KATA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// device address of the current device's scratch array
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* kata_status_string(kata_status_t status) {
  switch (status) {
    case KATA_OK: return "KATA_OK";
    case KATA_ERR_INVALID_VALUE: return "KATA_ERR_INVALID_VALUE";
    case KATA_ERR_UNSUPPORTED: return "KATA_ERR_UNSUPPORTED";
    case KATA_ERR_WORKSPACE: return "KATA_ERR_WORKSPACE";
    case KATA_ERR_DEVICE: return "KATA_ERR_DEVICE";
  }
  return "KATA_ERR_UNKNOWN";
}

int64_t kata_feature_dim(int d) { return d <= 0 ? -1 : static_cast<int64_t>(d) * (d + 1) / 2; }

kata_status_t kata_feature_map(const void* x, void* phi, int64_t rows, int d,
                               kata_dtype_t x_dtype, kata_dtype_t phi_dtype, void* stream) {
  if (x == nullptr || phi == nullptr) return KATA_ERR_INVALID_VALUE;
  if (rows <= 0 || d <= 0) return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(x_dtype) || !dtype_ok(phi_dtype)) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(phi)) return KATA_ERR_INVALID_VALUE;
  if (d > 64) return KATA_ERR_UNSUPPORTED;
  if (rows > (INT64_C(1) << 36)) return KATA_ERR_UNSUPPORTED;
  const int64_t D = kata_feature_dim(d);
  if (overlaps(x, rows * d * elem_size(x_dtype), phi, rows * D * elem_size(phi_dtype)))
    return KATA_ERR_INVALID_VALUE;
  return from_hip(kata::launch_feature_map(x, phi, rows, d, x_dtype == KATA_BF16,
                                           phi_dtype == KATA_BF16,
                                           static_cast<hipStream_t>(stream)));
}

size_t kata_forward_workspace_bytes(int B, int H, int64_t T, int d, int dv, int chunk,
                                    kata_scan_t scan) {
  // dtype does not change the workspace; plan with the larger-footprint path
  if (check_forward_shape(B, H, T, d, dv, chunk, KATA_BF16, scan) != KATA_OK) return 0;
  const ForwardPlan pb = kata::plan_forward(B, H, T, d, dv, chunk, KATA_BF16, scan);
  const ForwardPlan pf = kata::plan_forward(B, H, T, d, dv, chunk, KATA_F32, scan);
  return pb.ws_bytes > pf.ws_bytes ? pb.ws_bytes : pf.ws_bytes;
}

kata_status_t kata_forward_plan(int B, int H, int64_t T, int d, int dv, int chunk,
                                kata_dtype_t dtype, kata_scan_t scan, char* buf,
                                size_t buf_len) {
  const kata_status_t st = check_forward_shape(B, H, T, d, dv, chunk, dtype, scan);
  if (st != KATA_OK) return st;
  if (buf == nullptr || buf_len == 0) return KATA_ERR_INVALID_VALUE;
  const ForwardPlan p = kata::plan_forward(B, H, T, d, dv, chunk, dtype, scan);
  kata::describe_plan(p, buf, buf_len);
  return KATA_OK;
}

kata_status_t kata_forward_chunked(const void* q, const void* k, const void* v, void* out,
                                   int B, int H, int64_t T, int d, int dv, int chunk,
                                   float eps, kata_dtype_t dtype, kata_scan_t scan,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return kata_forward_chunked_profiled(q, k, v, out, B, H, T, d, dv, chunk, eps, dtype, scan,
                                       workspace, workspace_bytes, nullptr, stream);
}

kata_status_t kata_forward_quadratic(const void* q, const void* k, const void* v, void* out,
                                     int B, int H, int64_t T, int d, int dv, int g, float eps,
                                     kata_dtype_t dtype, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0 || g <= 0) return KATA_ERR_INVALID_VALUE;
  if (d % g != 0) return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!std::isfinite(eps) || eps < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KATA_ERR_INVALID_VALUE;
  if (!kata::quadratic_supported(dtype == KATA_BF16, d, dv, g)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  // one workgroup per (head, 128-query block): the grid must fit 2^31 - 1
  if (T > (INT64_C(1) << 40) / BH || BH * ((T + 127) / 128) > INT64_C(0x7fffffff))
    return KATA_ERR_UNSUPPORTED;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  if (overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes))
    return KATA_ERR_INVALID_VALUE;
  kata::QuadArgs a{q, k, v, out, BH, T, d, g, eps};
  return from_hip(kata::launch_forward_quadratic_mfma(a, static_cast<hipStream_t>(stream)));
}

size_t kata_forward_linear_workspace_bytes(int B, int H, int64_t T, int d, int dv, int chunk) {
  if (check_linear_shape(B, H, T, d, dv, chunk, KATA_FEATURE_ORTHANT, KATA_BF16) != KATA_OK) return 0;
  return plan_linear(static_cast<int64_t>(B) * H, T, chunk).ws_bytes;
}

kata_status_t kata_forward_linear(const void* q, const void* k, const void* v, void* out, int B,
                                  int H, int64_t T, int d, int dv, int chunk,
                                  kata_feature_t feature, float shift, float eps,
                                  kata_dtype_t dtype, kata_scan_t scan, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return KATA_ERR_INVALID_VALUE;
  const kata_status_t st = check_linear_shape(B, H, T, d, dv, chunk, feature, dtype);
  if (st != KATA_OK) return st;
  if (scan != KATA_SCAN_AUTO && scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE)
    return KATA_ERR_INVALID_VALUE;
  if (!std::isfinite(eps) || eps < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!std::isfinite(shift) || shift < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return KATA_ERR_INVALID_VALUE;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  if (overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes))
    return KATA_ERR_INVALID_VALUE;
  const LinPlan p = plan_linear(BH, T, chunk);
  if (p.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.ws_bytes) return KATA_ERR_WORKSPACE;
    if (overlaps(workspace, p.ws_bytes, out, v_bytes) || overlaps(workspace, p.ws_bytes, q, qk_bytes) ||
        overlaps(workspace, p.ws_bytes, k, qk_bytes) || overlaps(workspace, p.ws_bytes, v, v_bytes))
      return KATA_ERR_INVALID_VALUE;
  }
  if (BH * p.n_spans > INT64_C(0x7fffffff)) return KATA_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  kata::LinArgs a{q, k, v, out, static_cast<float*>(workspace), BH, T, static_cast<int>(feature),
                  shift, p.G, p.n_spans, eps, chunk};
  if (p.n_spans > 1) {
    hipError_t e = kata::launch_linear_span_state(a, s);
    // AUTO: sequential below 128 spans per head, reduce-then-scan from there
    const bool assoc = scan == KATA_SCAN_ASSOCIATIVE || (scan == KATA_SCAN_AUTO && p.n_spans >= 128);
    const int64_t E = kata::linear_state_floats(feature);
    if (e == hipSuccess) {
      e = assoc ? kata::launch_scan_associative(a.ws, BH, p.n_spans, E, s)
                : kata::launch_scan_sequential(a.ws, BH, p.n_spans, E, s);
    }
    if (e != hipSuccess) return KATA_ERR_DEVICE;
  }
  return from_hip(kata::launch_linear_readout(a, s));
}

size_t kata_forward_gated_workspace_bytes(int B, int H, int64_t T, int d, int dv, int chunk) {
  if (check_gated_shape(B, H, T, d, dv, chunk, KATA_BF16) != KATA_OK) return 0;
  return plan_gated(B, H, T, d, dv, chunk).bytes;
}

kata_status_t kata_forward_gated(const void* q, const void* k, const void* v, const float* log_gamma,
                                 void* out, int B, int H, int64_t T, int d, int dv, int chunk,
                                 kata_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || log_gamma == nullptr || out == nullptr)
    return KATA_ERR_INVALID_VALUE;
  const kata_status_t st = check_gated_shape(B, H, T, d, dv, chunk, dtype);
  if (st != KATA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_gamma) || !aligned16(out) ||
      !aligned16(workspace))
    return KATA_ERR_INVALID_VALUE;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  const size_t g_bytes = static_cast<size_t>(BH * T) * sizeof(float);
  if (overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes) || overlaps(out, v_bytes, log_gamma, g_bytes))
    return KATA_ERR_INVALID_VALUE;
  const GatedLayout l = plan_gated(B, H, T, d, dv, chunk);
  if (workspace == nullptr || workspace_bytes < l.bytes) return KATA_ERR_WORKSPACE;
  if (overlaps(workspace, l.bytes, out, v_bytes) || overlaps(workspace, l.bytes, q, qk_bytes) ||
      overlaps(workspace, l.bytes, k, qk_bytes) || overlaps(workspace, l.bytes, v, v_bytes) ||
      overlaps(workspace, l.bytes, log_gamma, g_bytes))
    return KATA_ERR_INVALID_VALUE;
  const ForwardPlan& p = l.p;
  if (BH * p.n_spans > INT64_C(0x7fffffff) || BH * p.n_chunks > (INT64_C(1) << 33))
    return KATA_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(workspace);
  float* gb = reinterpret_cast<float*>(wsb + l.gb_off);
  float* gk = reinterpret_cast<float*>(wsb + l.gk_off);
  float* ctot = reinterpret_cast<float*>(wsb + l.ctot_off);
  kata::MfmaArgs m{};
  m.q = q;
  m.k = k;
  m.v = v;
  m.out = out;
  m.ws = reinterpret_cast<float*>(wsb);
  m.BH = BH;
  m.T = T;
  m.d = d;
  m.chunk = chunk;
  m.G = p.G;
  m.n_spans = p.n_spans;
  m.eps = 0.f;
  m.gb = gb;
  m.gk = gk;
  hipError_t e = kata::launch_gate_prep(log_gamma, gb, gk, ctot, BH, T, chunk, s);
  if (e == hipSuccess && p.n_spans > 1) {
    e = kata::launch_span_state_gated(m, s);
    // the affine prefix: sequential below 128 spans per head, reduce-then-scan
    // from there (the additive prefix's measured crossover)
    if (e == hipSuccess) {
      e = p.n_spans >= 128
              ? kata::launch_scan_affine_associative(m.ws, ctot, BH, p.n_spans, p.E, p.G, p.n_chunks, s)
              : kata::launch_scan_affine(m.ws, ctot, BH, p.n_spans, p.E, p.G, p.n_chunks, s);
    }
  }
  if (e == hipSuccess) e = kata::launch_readout_gated(m, s);
  return from_hip(e);
}

kata_status_t kata_forward_chunked_profiled(const void* q, const void* k, const void* v,
                                            void* out, int B, int H, int64_t T, int d, int dv,
                                            int chunk, float eps, kata_dtype_t dtype,
                                            kata_scan_t scan, void* workspace,
                                            size_t workspace_bytes,
                                            const kata_stage_events_t* events, void* stream) {
  const kata_status_t st = check_forward_args(q, k, v, out, B, H, T, d, dv, chunk, eps, dtype, scan);
  if (st != KATA_OK) return st;
  if (!aligned16(workspace)) return KATA_ERR_INVALID_VALUE;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  const ForwardPlan p = kata::plan_forward(B, H, T, d, dv, chunk, dtype, scan);
  if (p.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.ws_bytes) return KATA_ERR_WORKSPACE;
    if (overlaps(workspace, p.ws_bytes, out, v_bytes) ||
        overlaps(workspace, p.ws_bytes, q, qk_bytes) ||
        overlaps(workspace, p.ws_bytes, k, qk_bytes) ||
        overlaps(workspace, p.ws_bytes, v, v_bytes))
      return KATA_ERR_INVALID_VALUE;
  }
  return from_hip(kata::run_forward(p, q, k, v, out, eps, static_cast<float*>(workspace),
                                    events, static_cast<hipStream_t>(stream)));
}

kata_status_t kata_forward_chunked_noalloc(const void* q, const void* k, const void* v, void* out,
                                           int B, int H, int64_t T, int d, int dv, int chunk,
                                           float eps, kata_dtype_t dtype, kata_scan_t scan,
                                           void* stream) {
  const kata_status_t st = check_forward_args(q, k, v, out, B, H, T, d, dv, chunk, eps, dtype, scan);
  if (st != KATA_OK) return st;
  const ForwardPlan p = kata::plan_forward(B, H, T, d, dv, chunk, dtype, scan);
  if (p.ws_bytes > KATA_NOALLOC_SCRATCH_BYTES) return KATA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.ws_bytes > 0 && scratch_address(&ws) != hipSuccess) return KATA_ERR_DEVICE;
  return from_hip(kata::run_forward(p, q, k, v, out, eps, static_cast<float*>(ws), nullptr,
                                    static_cast<hipStream_t>(stream)));
}

size_t kata_forward_chunked_blocks_workspace_bytes(int B, int H, int64_t T, int d, int dv, int g,
                                                   int chunk, kata_scan_t scan) {
  if (g == 1 && d != 64) return kata_forward_workspace_bytes(B, H, T, d, dv, chunk, scan);
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0 || g <= 0 || d % g != 0) return 0;
  if (scan != KATA_SCAN_AUTO && scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE) return 0;
  if (!kata::block_map_supported(true, d, dv, g, chunk)) return 0;
  if (T > (INT64_C(1) << 40) / (static_cast<int64_t>(B) * H)) return 0;
  return kata::plan_forward(B, H, T, d, dv, chunk, KATA_BF16, scan, g).ws_bytes;
}

kata_status_t kata_forward_chunked_blocks(const void* q, const void* k, const void* v, void* out,
                                          int B, int H, int64_t T, int d, int dv, int g, int chunk,
                                          float eps, kata_dtype_t dtype, kata_scan_t scan,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (g == 1 && d != 64)
    return kata_forward_chunked(q, k, v, out, B, H, T, d, dv, chunk, eps, dtype, scan, workspace,
                                workspace_bytes, stream);
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0 || chunk <= 0 || g <= 0 || d % g != 0)
    return KATA_ERR_INVALID_VALUE;
  if (scan != KATA_SCAN_AUTO && scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE)
    return KATA_ERR_INVALID_VALUE;
  if (!dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!kata::block_map_supported(dtype == KATA_BF16, d, dv, g, chunk)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH) return KATA_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return KATA_ERR_INVALID_VALUE;
  const size_t es = elem_size(dtype);
  const size_t qk_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  if (overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes))
    return KATA_ERR_INVALID_VALUE;
  const ForwardPlan p = kata::plan_forward(B, H, T, d, dv, chunk, dtype, scan, g);
  if (p.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.ws_bytes) return KATA_ERR_WORKSPACE;
    if (overlaps(workspace, p.ws_bytes, out, v_bytes) || overlaps(workspace, p.ws_bytes, q, qk_bytes) ||
        overlaps(workspace, p.ws_bytes, k, qk_bytes) || overlaps(workspace, p.ws_bytes, v, v_bytes))
      return KATA_ERR_INVALID_VALUE;
  }
  return from_hip(kata::run_forward(p, q, k, v, out, eps, static_cast<float*>(workspace), nullptr,
                                    static_cast<hipStream_t>(stream)));
}

kata_status_t kata_prefill_state(const void* k, const void* v, float* S, float* z, int B,
                                 int H, int64_t T, int d, int dv, kata_dtype_t dtype,
                                 void* stream) {
  if (k == nullptr || v == nullptr || S == nullptr || z == nullptr) return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || T <= 0 || !dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(z)) return KATA_ERR_INVALID_VALUE;
  if (!head_dim_ok(d) || !value_dim_ok(dv)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH || BH > (INT64_C(1) << 26)) return KATA_ERR_UNSUPPORTED;
  const int64_t D = kata_feature_dim(d);
  const size_t es = elem_size(dtype);
  const size_t s_bytes = static_cast<size_t>(BH * D * dv) * 4;
  const size_t z_bytes = static_cast<size_t>(BH * D) * 4;
  const size_t k_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  if (overlaps(S, s_bytes, z, z_bytes) || overlaps(S, s_bytes, k, k_bytes) ||
      overlaps(S, s_bytes, v, v_bytes) || overlaps(z, z_bytes, k, k_bytes) ||
      overlaps(z, z_bytes, v, v_bytes))
    return KATA_ERR_INVALID_VALUE;
  kata::StateArgs a{};
  a.k = k;
  a.v = v;
  a.S_out = S;
  a.z_out = z;
  a.BH = BH;
  a.T = T;
  a.d = d;
  a.dv = dv;
  a.span = T;
  a.n_spans = 1;
  a.s_stride = D * dv;
  a.z_stride = D;
  a.bf16 = dtype == KATA_BF16;
  a.sym = true;
  a.skip_last = false;
  return from_hip(kata::launch_state_valu(a, static_cast<hipStream_t>(stream)));
}

kata_status_t kata_prefill_state_gated(const void* k, const void* v, const float* log_gamma, float* S,
                                       int B, int H, int64_t T, int d, int dv, kata_dtype_t dtype,
                                       void* stream) {
  if (k == nullptr || v == nullptr || log_gamma == nullptr || S == nullptr) return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || T <= 0 || !dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(S) || (reinterpret_cast<uintptr_t>(log_gamma) & 3u) != 0)
    return KATA_ERR_INVALID_VALUE;
  if (!head_dim_ok(d) || !value_dim_ok(dv)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (T > (INT64_C(1) << 40) / BH || BH > (INT64_C(1) << 26)) return KATA_ERR_UNSUPPORTED;
  const int64_t D = kata_feature_dim(d);
  const size_t es = elem_size(dtype);
  const size_t s_bytes = static_cast<size_t>(BH * D * dv) * 4;
  const size_t k_bytes = static_cast<size_t>(BH * T * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * T * dv) * es;
  const size_t g_bytes = static_cast<size_t>(BH * T) * 4;
  if (overlaps(S, s_bytes, k, k_bytes) || overlaps(S, s_bytes, v, v_bytes) ||
      overlaps(S, s_bytes, log_gamma, g_bytes))
    return KATA_ERR_INVALID_VALUE;
  kata::StateArgs a{};
  a.k = k;
  a.v = v;
  a.S_out = S;
  a.z_out = nullptr;
  a.BH = BH;
  a.T = T;
  a.d = d;
  a.dv = dv;
  a.span = T;
  a.n_spans = 1;
  a.s_stride = D * dv;
  a.z_stride = 0;
  a.bf16 = dtype == KATA_BF16;
  a.sym = true;
  a.skip_last = false;
  a.log_gamma = log_gamma;
  return from_hip(kata::launch_state_valu(a, static_cast<hipStream_t>(stream)));
}

kata_status_t kata_decode_step(float* S, float* z, const void* q, const void* k,
                               const void* v, void* out, int B, int H, int d, int dv,
                               float eps, kata_dtype_t dtype, void* stream) {
  if (S == nullptr || z == nullptr || q == nullptr || k == nullptr || v == nullptr ||
      out == nullptr)
    return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || !dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!std::isfinite(eps) || eps < 0.f) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(out))
    return KATA_ERR_INVALID_VALUE;
  if (!head_dim_ok(d) || !value_dim_ok(dv)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > (INT64_C(1) << 30)) return KATA_ERR_UNSUPPORTED;
  const int64_t D = kata_feature_dim(d);
  const size_t es = elem_size(dtype);
  const size_t s_bytes = static_cast<size_t>(BH * D * dv) * 4;
  const size_t z_bytes = static_cast<size_t>(BH * D) * 4;
  const size_t qk_bytes = static_cast<size_t>(BH * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * dv) * es;
  if (overlaps(out, v_bytes, S, s_bytes) || overlaps(out, v_bytes, z, z_bytes) ||
      overlaps(out, v_bytes, q, qk_bytes) || overlaps(out, v_bytes, k, qk_bytes) ||
      overlaps(out, v_bytes, v, v_bytes) || overlaps(S, s_bytes, z, z_bytes))
    return KATA_ERR_INVALID_VALUE;
  return from_hip(kata::launch_decode(S, z, q, k, v, out, BH, d, dv, eps, dtype == KATA_BF16,
                                      static_cast<hipStream_t>(stream)));
}

kata_status_t kata_decode_step_gated(float* S, const void* q, const void* k, const void* v,
                                     const float* log_gamma, void* out, int B, int H, int d, int dv,
                                     kata_dtype_t dtype, void* stream) {
  if (S == nullptr || q == nullptr || k == nullptr || v == nullptr || log_gamma == nullptr ||
      out == nullptr)
    return KATA_ERR_INVALID_VALUE;
  if (B <= 0 || H <= 0 || !dtype_ok(dtype)) return KATA_ERR_INVALID_VALUE;
  if (!aligned16(S) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(log_gamma) & 3u) != 0)
    return KATA_ERR_INVALID_VALUE;
  if (!head_dim_ok(d) || !value_dim_ok(dv)) return KATA_ERR_UNSUPPORTED;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > (INT64_C(1) << 30)) return KATA_ERR_UNSUPPORTED;
  const int64_t D = kata_feature_dim(d);
  const size_t es = elem_size(dtype);
  const size_t s_bytes = static_cast<size_t>(BH * D * dv) * 4;
  const size_t qk_bytes = static_cast<size_t>(BH * d) * es;
  const size_t v_bytes = static_cast<size_t>(BH * dv) * es;
  const size_t g_bytes = static_cast<size_t>(BH) * 4;
  if (overlaps(out, v_bytes, S, s_bytes) || overlaps(out, v_bytes, q, qk_bytes) ||
      overlaps(out, v_bytes, k, qk_bytes) || overlaps(out, v_bytes, v, v_bytes) ||
      overlaps(out, v_bytes, log_gamma, g_bytes) || overlaps(S, s_bytes, log_gamma, g_bytes))
    return KATA_ERR_INVALID_VALUE;
  return from_hip(kata::launch_decode_gated(S, q, k, v, log_gamma, out, BH, d, dv, dtype == KATA_BF16,
                                            static_cast<hipStream_t>(stream)));
}

int64_t kata_probe_mfma_bf16(float* sink, int workgroups, int iters, void* stream) {
  if (sink == nullptr || !aligned16(sink) || workgroups <= 0 || iters <= 0) return -1;
  if (workgroups > (1 << 20) || iters > (1 << 24)) return -1;
  if (kata::launch_probe_mfma(sink, workgroups, iters, static_cast<hipStream_t>(stream)) != hipSuccess)
    return -1;
  return kata::probe_mfma_flops(workgroups, iters);
}

}  // extern "C"
