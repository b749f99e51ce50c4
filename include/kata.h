/*
 * kata.h -- C ABI of libkata: causal kernelized linear attention with the
 * rank-one PSD feature map, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "Kernelized Linear Attention: Breaking the Capacity
 * Wall with Symmetric Cones" (Ghriss & Chakraborty, arXiv 2607.17419), cited
 * below as "the KATA page".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) owned
 *    by the caller.  The library never allocates, frees or keeps device
 *    memory, and keeps no mutable global state; calls are reentrant.  The one
 *    exception is kata_forward_chunked_noalloc's static scratch array (below).
 *  - Tensors are dense, row-major, with the layouts stated per call.  Every
 *    pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is enqueued on it asynchronously; nothing synchronises.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error the call returns a status other than KATA_OK and has launched
 *    nothing and written nothing.  A failed launch returns KATA_ERR_DEVICE.
 *    Faults during execution surface at the caller's next synchronisation.
 *  - NaN/Inf inputs are not checked; they propagate.
 *  - Feature map: for x in R^d, phi(x) has D = d(d+1)/2 coordinates, the
 *    row-major upper triangle of x x^T, coordinate (i, j), i <= j, at index
 *    i*d - i*(i-1)/2 + (j - i), scaled by sqrt(2) when i != j, so that
 *    phi(q) . phi(k) = (q . k)^2 (the KATA page, Sec. 3.1 rank-one lift and
 *    Eq. 8 packed count).
 */
#ifndef KATA_H_
#define KATA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below are int-sized.  A C caller may pass any int where
 * one is expected (C allows values outside the enumerators); the C++
 * implementation gives them a fixed `int` base so that such a value is read
 * without undefined behaviour and rejected by validation. */
#ifdef __cplusplus
#define KATA_ENUM_BASE : int
#else
#define KATA_ENUM_BASE
#endif

typedef enum KATA_ENUM_BASE {
  KATA_F32 = 0,  /* IEEE binary32 */
  KATA_BF16 = 1  /* bfloat16 (upper half of binary32), round-to-nearest-even */
} kata_dtype_t;

typedef enum KATA_ENUM_BASE {
  KATA_SCAN_AUTO = 0,        /* library picks (measured default per shape) */
  KATA_SCAN_SEQUENTIAL = 1,  /* linear-depth pass over chunk states */
  KATA_SCAN_ASSOCIATIVE = 2, /* log-depth parallel scan over chunk states */
  KATA_SCAN_RECOMPUTE = 3,   /* no prefix pass: each readout workgroup sums the chunk
                                states before its span itself (kata_forward_chunked,
                                bf16, d = 16, dv = 64 only; no workspace) */
  KATA_SCAN_FUSED = 4        /* no prefix pass: the span sums are stored as by the
                                sequential pass and each readout workgroup adds
                                those of the spans before its own, in span order
                                (the sequential pass's sums, bit for bit);
                                kata_forward_chunked, bf16, dv = 64, d = 16 at
                                chunk 64 or 128, d = 32 at chunk 64 only */
} kata_scan_t;

typedef enum KATA_ENUM_BASE {
  KATA_OK = 0,
  KATA_ERR_INVALID_VALUE = 1, /* null pointer, non-positive size, bad eps, aliasing, misalignment */
  KATA_ERR_UNSUPPORTED = 2,   /* valid but outside the supported set (d, dv, chunk, dtype) */
  KATA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  KATA_ERR_DEVICE = 4         /* a HIP call or kernel launch failed */
} kata_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* kata_status_string(kata_status_t status);

/* Packed feature width D = d(d+1)/2 (the KATA page, Eq. 8); -1 if d <= 0. */
int64_t kata_feature_dim(int d);

/*
 * kata_feature_map -- phi(x) for `rows` vectors (the KATA page, Sec. 3.1:
 * psi(u) = u u^T, packed as described above).
 *   x   : [rows, d] in x_dtype
 *   phi : [rows, D] in phi_dtype (fp32 arithmetic, one rounding to phi_dtype)
 * Supported: 1 <= d <= 64, any rows >= 1.
 */
kata_status_t kata_feature_map(const void* x, void* phi, int64_t rows, int d,
                               kata_dtype_t x_dtype, kata_dtype_t phi_dtype,
                               void* stream);

/*
 * Bytes of device workspace kata_forward_chunked needs for this shape and
 * scan mode (0 on invalid arguments).  The workspace holds one fp32 state
 * pair (D x dv + D) per span of chunks the inter-chunk prefix runs over.
 */
size_t kata_forward_workspace_bytes(int B, int H, int64_t T, int d, int dv,
                                    int chunk, kata_scan_t scan);

/*
 * kata_forward_chunked -- causal normalised read with the rank-one PSD kernel,
 *   o_t = sum_{s<=t} (q_t.k_s)^2 v_s / (sum_{s<=t} (q_t.k_s)^2 + eps),
 * computed in the exact O(T) chunked-state form of the KATA page, Sec. 4.1
 * Eqs. 17-20 (per-chunk states phi(K_c)^T V_c and phi(K_c)^T 1, an exclusive
 * prefix over chunks, and per chunk the readout phi(Q_c) S_prefix plus the
 * causally masked (Q_c K_c^T)^2 block times V_c, normalised).  The prefix over
 * chunk states is the vector-space cumulative sum of Sec. 4.2, taken
 * sequentially, as a log-depth associative scan, or for heads of few spans
 * inside the readout (`scan`: KATA_SCAN_RECOMPUTE, KATA_SCAN_FUSED).
 *   q, k : [B, H, T, d] in dtype;  v, out : [B, H, T, dv] in dtype
 *   eps  : finite, >= 0; added once to the accumulated denominator
 *   chunk: chunk length C; a final partial chunk is zero-padded (App. D.2)
 * Arithmetic: KATA_F32 uses fp32 throughout; KATA_BF16 uses bf16 operands
 * with fp32 accumulation and fp32 normalisation, output rounded to bf16.
 * Supported: d in {16, 32}; dv in {16, 32, 64}; chunk in {32, 64, 128};
 * T >= 1; out must not overlap q, k or v; workspace_bytes >=
 * kata_forward_workspace_bytes(...) (workspace may be NULL when that is 0).
 * Deterministic for fixed arguments, scan mode and device.
 */
kata_status_t kata_forward_chunked(const void* q, const void* k, const void* v,
                                   void* out, int B, int H, int64_t T, int d,
                                   int dv, int chunk, float eps,
                                   kata_dtype_t dtype, kata_scan_t scan,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * kata_forward_chunked_noalloc -- kata_forward_chunked for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, kernels,
 * arguments, validation, status codes and output bits as kata_forward_chunked
 * with the same scan mode, but no workspace argument.  Its workspace is a
 * static device array of KATA_NOALLOC_SCRATCH_BYTES inside the library (each
 * device the library runs on holds its own copy until the process ends); the
 * call allocates nothing and calls no allocating routine.
 *   - A shape whose workspace (kata_forward_workspace_bytes) exceeds
 *     KATA_NOALLOC_SCRATCH_BYTES returns KATA_ERR_WORKSPACE before anything
 *     is enqueued (the T = 131072, 8-head, d = 16 forward needs 19.2 MB).
 *   - Every call on a device shares that device's array and leaves its last
 *     contents there (nothing in it needs to start at zero).  Calls that
 *     overlap in time on one device -- concurrent streams, or host threads
 *     without ordering between their streams -- race on it and must not be
 *     issued; calls ordered on one stream are safe.
 *   - The first call on each device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current; a failure there
 *     returns KATA_ERR_DEVICE.
 */
#define KATA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kata_status_t kata_forward_chunked_noalloc(const void* q, const void* k, const void* v,
                                           void* out, int B, int H, int64_t T, int d,
                                           int dv, int chunk, float eps,
                                           kata_dtype_t dtype, kata_scan_t scan,
                                           void* stream);

/*
 * kata_forward_quadratic -- the causal read of kata_forward_chunked,
 *   o_t = sum_{s<=t} c_{t,s} v_s / (sum_{s<=t} c_{t,s} + eps),
 * evaluated in its direct O(T^2) form: the read of the KATA page, Eq. 2, which
 * the page runs as its quadratic operating point beside the chunked one
 * (Sec. 4, Table 8).  The score is that of the KATA-Mg block maps (Sec. 4.1):
 * q and k split into g equal blocks of width m = d/g and
 *   c_{t,s} = sum_a (q_{t,a} . k_{s,a})^2,
 * which at g = 1 is the full rank-one lift's (q_t . k_s)^2 (Sec. 3.1).  Per
 * block of 128 queries, every key block up to the diagonal contributes its
 * causally masked scores times [V | 1]; there is no state and no workspace.
 * The work grows as T^2: it is the faster form for short T.
 *   q, k : [B, H, T, d] bf16;  v, out : [B, H, T, dv] bf16
 *   g    : feature blocks, >= 1, dividing d (1 = the full map)
 *   eps  : finite, >= 0; added once to the accumulated denominator
 * Arithmetic: bf16 operands, fp32 scores, squares and accumulation, scores
 * rounded to bf16 before they weight V, fp32 normalisation, output rounded to
 * bf16.
 * Supported: KATA_BF16; dv = 64; d in {16, 32, 64} with block width d/g in
 * {16, 32, 64} (M1, M2, M4 at d = 64); T >= 1 (other shapes and KATA_F32
 * return KATA_ERR_UNSUPPORTED; g < 1 or g not dividing d is
 * KATA_ERR_INVALID_VALUE).  Pointers 16-byte aligned; out must not overlap q,
 * k or v.  Deterministic for fixed arguments and device.
 */
kata_status_t kata_forward_quadratic(const void* q, const void* k, const void* v,
                                     void* out, int B, int H, int64_t T, int d,
                                     int dv, int g, float eps, kata_dtype_t dtype,
                                     void* stream);

/*
 * kata_forward_gated -- the gated read of the KATA page's GatedKATA (App.
 * F.4): the state decays by a per-token scalar gate before each write,
 *   S_t = gamma_t S_{t-1} + phi(k_t) v_t^T,   o_t = phi(q_t)^T S_t,
 * with no denominator, i.e. o_t = sum_{s<=t} (prod_{r=s+1..t} gamma_r)
 * (q_t.k_s)^2 v_s (the unrolled form of Sec. 5.2), phi the rank-one lift.
 * Computed chunkwise like kata_forward_chunked: per chunk the running sums
 * b_t of log gamma from the chunk start weight the intra-chunk scores by
 * exp(b_t - b_s), the incoming state by exp(b_t), and the keys written to the
 * state by exp(b_C - b_s); the prefix over span states is affine (each span's
 * state scaled by its gate product before the next is added).
 *   q, k      : [B, H, T, d] bf16;  v, out : [B, H, T, dv] bf16
 *   log_gamma : [B, H, T] fp32, log of the gate (expected <= 0: the page's
 *               gate is a sigmoid; larger values can overflow)
 *   chunk     : chunk length, 64 or 128
 * Arithmetic: gate sums in fp32 (log2 units), bf16 operands, fp32 scores,
 * states and accumulation, bf16 output.
 * Supported: KATA_BF16, d in {16, 32}, dv = 64, T >= 1 (other shapes and
 * KATA_F32 return KATA_ERR_UNSUPPORTED).  The workspace is always needed:
 * workspace_bytes >= kata_forward_gated_workspace_bytes(...).  Pointers
 * 16-byte aligned; out and the workspace must not overlap each other or the
 * inputs.  Deterministic for fixed arguments and device.
 */
size_t kata_forward_gated_workspace_bytes(int B, int H, int64_t T, int d, int dv,
                                          int chunk);
kata_status_t kata_forward_gated(const void* q, const void* k, const void* v,
                                 const float* log_gamma, void* out, int B, int H,
                                 int64_t T, int d, int dv, int chunk,
                                 kata_dtype_t dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * kata_forward_chunked_blocks -- the chunked read of kata_forward_chunked with
 * the KATA-Mg block maps of the KATA page (Sec. 4.1): q and k split into g
 * equal blocks of width m = d/g, psi_Mg(u) = (u_1 u_1^T, ..., u_g u_g^T), so
 *   o_t = sum_{s<=t} c_{t,s} v_s / (sum_{s<=t} c_{t,s} + eps),
 *   c_{t,s} = sum_a (q_{t,a} . k_{s,a})^2,
 * in the same O(T) chunked-state form (Eqs. 17-20) with the g m(m+1)/2
 * block features.  g = 1 is exactly kata_forward_chunked (and takes its
 * supported set); the block map g = 4 is supported at d = 64 (KATA-M4, 544
 * features), bf16, dv = 64, chunk 64.  Arguments, workspace, errors and
 * determinism as kata_forward_chunked; workspace_bytes >=
 * kata_forward_chunked_blocks_workspace_bytes(...).
 */
size_t kata_forward_chunked_blocks_workspace_bytes(int B, int H, int64_t T, int d,
                                                   int dv, int g, int chunk,
                                                   kata_scan_t scan);
kata_status_t kata_forward_chunked_blocks(const void* q, const void* k, const void* v,
                                          void* out, int B, int H, int64_t T, int d,
                                          int dv, int g, int chunk, float eps,
                                          kata_dtype_t dtype, kata_scan_t scan,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/* Linear (D = d) features of kata_forward_linear. */
typedef enum KATA_ENUM_BASE {
  KATA_FEATURE_ORTHANT = 0,  /* psi(x) = ReLU(x) + shift, every coordinate */
  KATA_FEATURE_LORENTZ = 1,  /* psi(x) = (y, |y|_2 (1 + s^2)), y = x_{1..d-1}, s = x_d */
  KATA_FEATURE_IDENTITY = 2  /* psi(x) = x; read without a denominator (see below) */
} kata_feature_t;

/*
 * kata_forward_linear -- the causal read with a linear (D = d) feature psi
 * instead of the rank-one lift, c_{t,s} = psi(q_t) . psi(k_s):
 *   cone maps (KATA-Orthant, KATA-Lorentz of the KATA page, App. F.4; the
 *   two cone families of Sec. 2.3), whose scores are never negative, read
 *   normalised:  o_t = sum_{s<=t} c_{t,s} v_s / (sum_{s<=t} c_{t,s} + eps);
 *   the identity map psi(x) = x, the first-order workload of the page's
 *   associative-scan tables (Sec. 4.2, Tables 10-11, a d x dv state), has
 *   signed scores and is read without a denominator:
 *                o_t = sum_{s<=t} (q_t . k_s) v_s   (shift and eps unused).
 * Computed in the chunked form of Sec. 4.1 Eqs. 17-20 with D = d: per-span
 * states psi(K)^T [V | 1], an exclusive prefix over spans (Sec. 4.2),
 * sequential or log-depth associative (`scan`; AUTO takes the associative
 * one from 128 spans per head), and per chunk psi(Q) [S | z] plus the
 * causally masked psi(Q) psi(K)^T block times [V | 1].
 *   q, k : [B, H, T, d] bf16;  v, out : [B, H, T, dv] bf16
 *   chunk: chunk length, 32, 64 or 128; a final partial chunk is zero-padded
 *   shift: the orthant map's shift, finite, >= 0 (ignored by the others)
 *   eps  : finite, >= 0; added once to the accumulated denominator
 * Arithmetic: psi computed in fp32 from the bf16 inputs and rounded to bf16;
 * fp32 scores, states and accumulation; scores and the readout's state copy
 * rounded to bf16 before they multiply; fp32 normalisation; bf16 output.
 * Supported: KATA_BF16, d = 64, dv = 64, chunk in {32, 64, 128}, T >= 1
 * (other shapes and KATA_F32 return KATA_ERR_UNSUPPORTED).  workspace_bytes
 * >= kata_forward_linear_workspace_bytes(...) (workspace may be NULL when
 * that is 0).  Pointers 16-byte aligned; out and the workspace must not
 * overlap each other or the inputs.  Deterministic for fixed arguments, scan
 * mode and device.
 */
size_t kata_forward_linear_workspace_bytes(int B, int H, int64_t T, int d, int dv,
                                           int chunk);
kata_status_t kata_forward_linear(const void* q, const void* k, const void* v,
                                  void* out, int B, int H, int64_t T, int d, int dv,
                                  int chunk, kata_feature_t feature, float shift,
                                  float eps, kata_dtype_t dtype, kata_scan_t scan,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Optional profiling hook: hipEvent_t handles (as void*) recorded on `stream`
 * immediately before and after each stage of kata_forward_chunked -- stage 0
 * the span-state sums, stage 1 the prefix over spans, stage 2 the chunked
 * readout.  A stage the plan does not run gets its two events recorded back
 * to back.  NULL entries are skipped.  The events are caller-owned.
 */
typedef struct {
  void* stage_begin[3];
  void* stage_end[3];
} kata_stage_events_t;

/*
 * kata_forward_chunked_profiled -- kata_forward_chunked, additionally
 * recording the stage events in `events` (may be NULL).  Same contract,
 * validation and results.
 */
kata_status_t kata_forward_chunked_profiled(const void* q, const void* k, const void* v,
                                            void* out, int B, int H, int64_t T, int d,
                                            int dv, int chunk, float eps,
                                            kata_dtype_t dtype, kata_scan_t scan,
                                            void* workspace, size_t workspace_bytes,
                                            const kata_stage_events_t* events,
                                            void* stream);

/*
 * kata_prefill_state -- recurrent state of a history, for decoding:
 *   S = sum_t phi(k_t) v_t^T   [B*H, D, dv] fp32 (row-major, dv contiguous)
 *   z = sum_t phi(k_t)         [B*H, D]     fp32
 * (the KATA page, Sec. 2: S_t and Z_t of Eq. 2), with the sqrt(2)-weighted
 * packing above.  k : [B, H, T, d], v : [B, H, T, dv] in dtype.  S and z are
 * overwritten.  Supported: d in {16, 32}; dv in {16, 32, 64}; T >= 1.
 */
kata_status_t kata_prefill_state(const void* k, const void* v, float* S,
                                 float* z, int B, int H, int64_t T, int d,
                                 int dv, kata_dtype_t dtype, void* stream);

/*
 * kata_prefill_state_gated -- GatedKATA state of a history, for continuing
 * it with kata_decode_step_gated (the KATA page, App. F.4: S_t = gamma_t
 * S_{t-1} + psi(k_t) v_t^T from S_0 = 0; unrolled, Sec. 5.2):
 *   S = sum_t (prod_{r=t+1..T} gamma_r) phi(k_t) v_t^T   [B*H, D, dv] fp32
 * in the layout of kata_prefill_state (no z: the gated read has no
 * denominator), taken token by token in fp32.
 *   k : [B, H, T, d], v : [B, H, T, dv] in dtype
 *   log_gamma : [B, H, T] fp32, log of the gate per token (4-byte aligned)
 * S is overwritten.  Supported: d in {16, 32}; dv in {16, 32, 64}; T >= 1.
 * S must not overlap the inputs.
 */
kata_status_t kata_prefill_state_gated(const void* k, const void* v, const float* log_gamma,
                                       float* S, int B, int H, int64_t T, int d, int dv,
                                       kata_dtype_t dtype, void* stream);

/*
 * kata_decode_step -- one token of the additive recurrence (the KATA page,
 * Sec. 2: S_t = S_{t-1} + psi(k_t) v_t^T, Z_t = Z_{t-1} + psi(k_t)), then
 * the normalised read including that token:
 *   S += phi(k) v^T;  z += phi(k);  out = phi(q)^T S / (phi(q)^T z + eps).
 *   S    : [B*H, D, dv] fp32, updated in place (layout as kata_prefill_state)
 *   z    : [B*H, D]     fp32, updated in place
 *   q, k : [B*H, d] in dtype;  v, out : [B*H, dv] in dtype
 * fp32 arithmetic.  Supported: d in {16, 32}; dv in {16, 32, 64}.
 * out must not overlap S, z, q, k or v.
 */
kata_status_t kata_decode_step(float* S, float* z, const void* q,
                               const void* k, const void* v, void* out,
                               int B, int H, int d, int dv, float eps,
                               kata_dtype_t dtype, void* stream);

/*
 * kata_decode_step_gated -- one token of the GatedKATA recurrence (the KATA
 * page, App. F.4: S_t = gamma_t S_{t-1} + psi(k_t) v_t^T, read
 * o_t = psi(q_t)^T S_t with no denominator), read after the update:
 *   S = exp(log_gamma) S + phi(k) v^T;  out = phi(q)^T S.
 *   S         : [B*H, D, dv] fp32, updated in place (layout as kata_prefill_state)
 *   q, k      : [B*H, d] in dtype;  v, out : [B*H, dv] in dtype
 *   log_gamma : [B*H] fp32, the step's log gate per head (4-byte aligned)
 * fp32 arithmetic.  Supported: d in {16, 32}; dv in {16, 32, 64}.
 * out must not overlap S, q, k, v or log_gamma.
 */
kata_status_t kata_decode_step_gated(float* S, const void* q, const void* k,
                                     const void* v, const float* log_gamma,
                                     void* out, int B, int H, int d, int dv,
                                     kata_dtype_t dtype, void* stream);

/*
 * kata_forward_plan -- describe the launch plan kata_forward_chunked uses for
 * these arguments as a one-line text (kernels, chunk span per prefix entry,
 * grid sizes) into buf (NUL-terminated, truncated to buf_len).  Returns the
 * same status kata_forward_chunked's validation would, minus pointer checks.
 */
kata_status_t kata_forward_plan(int B, int H, int64_t T, int d, int dv,
                                int chunk, kata_dtype_t dtype,
                                kata_scan_t scan, char* buf, size_t buf_len);

/*
 * kata_probe_mfma_bf16 -- measurement aid, not part of the method: the
 * device's dense bf16 matrix-core rate, for reporting measured peaks beside
 * the datasheet ones.  Launches `workgroups` workgroups of 4 waves on
 * `stream`; each wave runs `iters` rounds of 8 independent 16x16x32 bf16
 * products with fp32 accumulation on constant operands, and every thread
 * writes one fp32 sum to sink (device, caller-owned, >= workgroups * 256
 * floats, 16-byte aligned; its values carry no meaning).  Returns the FLOP
 * count of the launch (workgroups * 4 * iters * 8 * 16384), to be divided by
 * the launch's duration between events on `stream`, or -1 for a null or
 * misaligned sink, workgroups outside [1, 2^20], iters outside [1, 2^24], or
 * a launch error.
 */
int64_t kata_probe_mfma_bf16(float* sink, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KATA_H_ */
