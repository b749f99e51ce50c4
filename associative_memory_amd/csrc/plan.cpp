#include "plan.h"

#include <cstdio>

#include "kernels.h"
#include "plan_mfma.h"

namespace kata {
namespace {

constexpr int64_t kValuDvTile = 16;
constexpr int64_t kMaxSpans = 8192;     // the gated affine prefix keeps span decays in LDS
constexpr int64_t kTargetWorkgroups = 2048;
// resident readout workgroups per CU: two of 4 waves at d = 16, one of 8 at d = 32
constexpr int64_t mfma_target_workgroups(int d) { return d == 16 ? 512 : 256; }
// paired spans at d = 16: the even span of a pair takes G + G / kPairSkewDiv
// chunks and runs in the readout workgroup placed first on its CU, which
// issues ahead of the second (measured at 8 heads x 64 spans of 16 chunks:
// readout 84 -> 81 us, span sums 38 -> 37 us)
constexpr int64_t kPairSkewDiv = 8;
// d = 16 matrix-core path: spans of at least this many tokens, as long as
// the readout keeps one workgroup per CU.  Below it a span's 37 KB state
// (written, scanned, read back) costs more than the extra workgroups give
// (B=4 H=8 T=2048, chunk 64 / 128: 16 spans per head 30.4 / 31.4 us, 8 spans
// 28.7 / 28.5 us, 4 spans 34.7 / 31.0 us); from T = 8192 on the workgroup
// target already gives spans of 256 tokens or more.
constexpr int64_t kMinSpanTokens16 = 256;
constexpr int64_t kMinReadoutWorkgroups16 = 256;
// prefix formed in the readout workgroups: about this many workgroups, and
// the automatic choice only while the latest span carries at most this many
// tokens before it (measured, step us, sequential prefix / recompute:
// B=4 H=8 d=16 bf16, T=512 C=64 21.4 / 10.4, T=1024 C=64 29.1 / 17.0,
// T=1024 C=128 23.5 / 14.8; B=16 H=16 T=1024 C=64 46.6 / 30.3; at 1,800 to
// 1,900 tokens before the latest span the two are within 10% either way:
// B=4 H=8 T=2048 C=128 28.0 / 26.0, C=64 27.7 / 29.8, B=1 H=8 T=2048 C=128
// 18.4 / 22.5; beyond, the recompute loses: B=4 H=8 T=4096 C=128 37.1 / 48.9)
constexpr int64_t kRecomputeWorkgroups = 512;
constexpr int64_t kRecomputeMaxPrefixTokens = 1024;
// prefix added in the readout workgroups from the stored span sums (no
// prefix launch): the automatic choice at d = 16 up to this many spans per
// head (measured, step us, sequential / recompute / fused, d = 16 bf16
// chunk 64: B=4 H=8 T=2048 (8 spans) 26.8 / 26.2 / 22.6, B=8 H=8 T=2048
// 33.6 / 28.7 / 27.3, B=4 H=8 T=4096 (16 spans) 34.2 / 47.6 / 30.9;
// B=2 H=8 T=8192 (32 spans) 34.7 / 85.7 / 39.7, B=1 H=8 T=16384 (64)
// 34.9 / 161.6 / 57.6)
constexpr int64_t kFusedMaxSpans = 16;
// the same at d = 32 (137 KB span states; step us, sequential / fused,
// B x H x T, chunk 64: 8 x 16 x 2048 (2 spans) 103.4 / 84.9, 8 x 16 x 4096
// (2) 167.0 / 148.3, 4 x 16 x 2048 (4) 73.3 / 65.7, 4 x 16 x 4096 (4)
// 106.3 / 98.1; 4 x 8 x 4096 (8) 74.5 / 91.3, 2 x 16 x 8192 (8) 106.9 / 122.7)
constexpr int64_t kFusedMaxSpans32 = 4;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

ForwardPlan plan_forward(int B, int H, int64_t T, int d, int dv, int chunk,
                         kata_dtype_t dtype, kata_scan_t scan, int g) {
  ForwardPlan p;
  p.BH = static_cast<int64_t>(B) * H;
  p.T = T;
  p.d = d;
  p.dv = dv;
  p.chunk = chunk;
  p.D = d * (d + 1) / 2;
  p.bf16 = dtype == KATA_BF16;
  p.n_chunks = ceil_div(T, chunk);
  const bool blocks = d == 64 && block_map_supported(p.bf16, d, dv, g, chunk);
  const bool mfma = mfma_supported(p.bf16, d, dv, chunk) || blocks;
  if (blocks && g != 4) {
    p.nsl = g == 1 ? 4 : 2;
    p.fm_base = g == 1 ? 100 : 200;
  }
  p.path = mfma ? Path::Mfma : Path::Valu;
  p.E = mfma ? mfma_state_floats(d) : static_cast<int64_t>(p.D) * dv + p.D;

  if (scan == KATA_SCAN_RECOMPUTE || scan == KATA_SCAN_AUTO) {
    // every readout workgroup sums the chunks before its span itself
    int64_t spans = ceil_div(kRecomputeWorkgroups, p.BH);
    if (spans > p.n_chunks) spans = p.n_chunks;
    const int64_t G = ceil_div(p.n_chunks, spans);
    const bool short_prefix = (p.n_chunks - G) * chunk <= kRecomputeMaxPrefixTokens;
    if (scan == KATA_SCAN_RECOMPUTE ||
        (short_prefix && recompute_supported(p.bf16, d, dv, chunk) && g == 1)) {
      p.scan = KATA_SCAN_RECOMPUTE;
      p.G = G;
      p.n_spans = ceil_div(p.n_chunks, p.G);
      p.wg_output = p.BH * p.n_spans;
      return p;
    }
  }
  const int64_t tiles = mfma ? 1 : dv / kValuDvTile;
  // enough spans to give the readout about the target number of workgroups
  int64_t spans = ceil_div(mfma ? mfma_target_workgroups(d) : kTargetWorkgroups, p.BH * tiles);
  if (spans > p.n_chunks) spans = p.n_chunks;
  if (mfma && d == 16 && spans > T / kMinSpanTokens16 && T >= kMinSpanTokens16) {
    const int64_t cap = T / kMinSpanTokens16;
    if (ceil_div(p.n_chunks, ceil_div(p.n_chunks, cap)) * p.BH >= kMinReadoutWorkgroups16) spans = cap;
  }
  if (spans < 1) spans = 1;
  p.G = ceil_div(p.n_chunks, spans);
  if (ceil_div(p.n_chunks, p.G) > kMaxSpans) p.G = ceil_div(p.n_chunks, kMaxSpans);
  p.n_spans = ceil_div(p.n_chunks, p.G);
  // few heads at short T: rather than more spans than the fused prefix takes
  // (and a prefix launch), kFusedMaxSpans spans of at most kMinSpanTokens16
  // tokens (measured, step us, B x H x T chunk, as planned before / capped:
  // 2x8x2048 C64 (32 spans) 28.5 / 21.8, 1x8x4096 C64 (64) 28.6 / 24.0,
  // 2x8x4096 C64 and 1x16x4096 C64 (32) equal; with longer capped spans the
  // cap loses: 1x8x8192 C128 27.5 / 29.9, 1x8x16384 C128 36.3 / 44.3)
  if (scan == KATA_SCAN_AUTO && mfma && d == 16 && g == 1 && p.n_spans > kFusedMaxSpans &&
      ceil_div(p.n_chunks, kFusedMaxSpans) * chunk <= kMinSpanTokens16 &&
      fused_supported(p.bf16, d, dv, chunk)) {
    p.G = ceil_div(p.n_chunks, kFusedMaxSpans);
    p.n_spans = ceil_div(p.n_chunks, p.G);
  }
  if (scan == KATA_SCAN_AUTO) {
    // measured on MI355X at 9,360-float span states (prefix stage, us,
    // sequential / associative): 8 heads x 64 spans 11.2 / 11.7, 4 x 128
    // 12.7 / 12.4, 1 x 512 29.8 / 19.6; d = 32, 32 x 8 spans 14.4 / 15.1
    if (p.n_spans > 1 && p.n_spans <= (d == 16 ? kFusedMaxSpans : kFusedMaxSpans32) && g == 1 &&
        fused_supported(p.bf16, d, dv, chunk)) {
      scan = KATA_SCAN_FUSED;
    } else {
      scan = p.n_spans >= 128 ? KATA_SCAN_ASSOCIATIVE : KATA_SCAN_SEQUENTIAL;
    }
  }
  // (the fused prefix maps spans to workgroups by head, without pairs)
  if (mfma && d == 16 && p.n_spans % 2 == 0 && p.n_chunks == p.n_spans * p.G &&
      p.G >= kPairSkewDiv && p.n_spans * p.BH == mfma_target_workgroups(d) && scan != KATA_SCAN_FUSED)
    p.GL = p.G + p.G / kPairSkewDiv;
  p.scan = scan;
  p.wg_output = p.BH * p.n_spans * tiles;
  if (p.n_spans > 1) {
    p.wg_state = p.BH * (mfma ? p.n_spans - 1 : p.n_spans) * tiles * p.nsl;
    p.ws_bytes = static_cast<size_t>(p.nsl * p.BH * p.n_spans * p.E) * sizeof(float);
  }
  if (p.nsl > 1) {
    p.part_off = (p.ws_bytes + 255) & ~static_cast<size_t>(255);
    p.ws_bytes = p.part_off + static_cast<size_t>(p.BH * T * kPartFloats) * sizeof(float);
  }
  return p;
}

void describe_plan(const ForwardPlan& p, char* buf, size_t len) {
  std::snprintf(buf, len,
                "path=%s scan=%s D=%d chunk=%d n_chunks=%lld chunks_per_span=%lld "
                "paired_even_span=%lld n_spans=%lld wg_state=%lld wg_output=%lld "
                "workspace_bytes=%zu",
                p.path == Path::Mfma ? "mfma" : "valu",
                p.scan == KATA_SCAN_ASSOCIATIVE ? "associative"
                : p.scan == KATA_SCAN_RECOMPUTE ? "recompute"
                : p.scan == KATA_SCAN_FUSED     ? "fused"
                                                : "sequential",
                p.D, p.chunk,
                static_cast<long long>(p.n_chunks), static_cast<long long>(p.G),
                static_cast<long long>(p.GL),
                static_cast<long long>(p.n_spans), static_cast<long long>(p.wg_state),
                static_cast<long long>(p.wg_output), p.ws_bytes);
}

namespace {

hipError_t mark(const kata_stage_events_t* ev, bool begin, int stage, hipStream_t stream) {
  if (ev == nullptr) return hipSuccess;
  void* h = begin ? ev->stage_begin[stage] : ev->stage_end[stage];
  if (h == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(h), stream);
}

}  // namespace

hipError_t run_forward(const ForwardPlan& p, const void* q, const void* k, const void* v,
                       void* out, float eps, float* ws, const kata_stage_events_t* ev,
                       hipStream_t stream) {
  hipError_t e = hipSuccess;
#define KATA_TRY(x)                  \
  do {                               \
    e = (x);                         \
    if (e != hipSuccess) return e;   \
  } while (0)
  KATA_TRY(mark(ev, true, 0, stream));
  if (p.path == Path::Mfma && p.nsl > 1) {
    // sliced feature map: span sums per slice, one prefix over every slice's
    // heads, then the slices' readouts in order (each adds to the fp32 partial
    // reads; the last normalises)
    MfmaArgs m{};
    m.q = q;
    m.k = k;
    m.v = v;
    m.out = out;
    m.BH = p.BH;
    m.T = p.T;
    m.d = p.d;
    m.chunk = p.chunk;
    m.G = p.G;
    m.n_spans = p.n_spans;
    m.eps = eps;
    m.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_off);
    const int64_t slice_floats = p.BH * p.n_spans * p.E;
    if (p.n_spans > 1) {
      for (int s = 0; s < p.nsl; ++s) {
        m.fm = p.fm_base + s;
        m.ws = ws + s * slice_floats;
        KATA_TRY(launch_span_state_mfma(m, stream));
      }
      KATA_TRY((p.scan == KATA_SCAN_ASSOCIATIVE)
                   ? launch_scan_associative(ws, p.nsl * p.BH, p.n_spans, p.E, stream)
                   : launch_scan_sequential(ws, p.nsl * p.BH, p.n_spans, p.E, stream));
    }
    for (int s = 0; s < p.nsl; ++s) {
      m.fm = p.fm_base + s;
      m.ws = p.n_spans > 1 ? ws + s * slice_floats : nullptr;
      KATA_TRY(launch_readout_mfma(m, stream));
    }
    return hipSuccess;
  }
  if (p.path == Path::Mfma) {
    MfmaArgs m{};
    m.q = q;
    m.k = k;
    m.v = v;
    m.out = out;
    m.ws = ws;
    m.BH = p.BH;
    m.T = p.T;
    m.d = p.d;
    m.chunk = p.chunk;
    m.G = p.G;
    m.GL = p.GL;
    m.n_spans = p.n_spans;
    m.eps = eps;
    m.recompute = p.scan == KATA_SCAN_RECOMPUTE;
    m.fused = p.scan == KATA_SCAN_FUSED;
    if (p.n_spans > 1 && !m.recompute) KATA_TRY(launch_span_state_mfma(m, stream));
    KATA_TRY(mark(ev, false, 0, stream));
    KATA_TRY(mark(ev, true, 1, stream));
    if (p.n_spans > 1 && !m.recompute && !m.fused) {
      KATA_TRY((p.scan == KATA_SCAN_ASSOCIATIVE)
                   ? launch_scan_associative(ws, p.BH, p.n_spans, p.E, stream)
                   : launch_scan_sequential(ws, p.BH, p.n_spans, p.E, stream));
    }
    KATA_TRY(mark(ev, false, 1, stream));
    KATA_TRY(mark(ev, true, 2, stream));
    KATA_TRY(launch_readout_mfma(m, stream));
    KATA_TRY(mark(ev, false, 2, stream));
    return hipSuccess;
  }
  if (p.n_spans > 1) {
    StateArgs s{};
    s.k = k;
    s.v = v;
    s.S_out = ws;
    s.z_out = ws + static_cast<int64_t>(p.D) * p.dv;
    s.BH = p.BH;
    s.T = p.T;
    s.d = p.d;
    s.dv = p.dv;
    s.span = p.G * p.chunk;
    s.n_spans = p.n_spans;
    s.s_stride = p.E;
    s.z_stride = p.E;
    s.bf16 = p.bf16;
    s.sym = false;
    s.skip_last = true;
    KATA_TRY(launch_state_valu(s, stream));
    KATA_TRY(mark(ev, false, 0, stream));
    KATA_TRY(mark(ev, true, 1, stream));
    KATA_TRY((p.scan == KATA_SCAN_ASSOCIATIVE)
                 ? launch_scan_associative(ws, p.BH, p.n_spans, p.E, stream)
                 : launch_scan_sequential(ws, p.BH, p.n_spans, p.E, stream));
  } else {
    KATA_TRY(mark(ev, false, 0, stream));
    KATA_TRY(mark(ev, true, 1, stream));
  }
  KATA_TRY(mark(ev, false, 1, stream));
  OutputArgs o{};
  o.q = q;
  o.k = k;
  o.v = v;
  o.out = out;
  o.prefix = p.n_spans > 1 ? ws : nullptr;
  o.BH = p.BH;
  o.T = p.T;
  o.d = p.d;
  o.dv = p.dv;
  o.chunk = p.chunk;
  o.G = p.G;
  o.n_spans = p.n_spans;
  o.eps = eps;
  o.bf16 = p.bf16;
  KATA_TRY(mark(ev, true, 2, stream));
  KATA_TRY(launch_output_valu(o, stream));
  KATA_TRY(mark(ev, false, 2, stream));
#undef KATA_TRY
  return hipSuccess;
}

}  // namespace kata
