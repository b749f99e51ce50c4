// Helpers shared by the matrix-core kernels of libkata (bf16 MFMA with fp32
// accumulation on gfx950): vector types, the 16x16x32 / 16x16x16 products,
// buffer resources with hardware range checks, LDS DMA and the transposing
// LDS read, wait-count and barrier helpers, and per-wave specialisation.
// Everything is internal to each kernel source (anonymous namespace).
#pragma once

#include <utility>

#include "common.h"
#include "plan_mfma.h"

namespace kata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int DV = 64;
constexpr int NDT = kMfmaValueTiles;  // 4 value tiles + the ones-column tile
// LDS rows of V^T and of the state copy: 64 value rows, then row 64 (ones
// for V, z for the state) and row 65 (zeros).  Operand rows 65..79 of the
// ones-column tile are all zero, so every lane past the first reads row 65.
constexpr int VROWS = DV + 2;
__device__ __forceinline__ int vrow(int vt, int r) { return vt == NDT - 1 ? DV + (r > 0) : 16 * vt + r; }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ small helpers

// Calls f(std::integral_constant<int, W>) for the wave index w (uniform per
// wave): each wave runs a body specialised for its index, so the per-wave
// work split (query tiles, feature tiles, lane rotations) is resolved at
// compile time and the chunk body has no wave-dependent branches.
template <int NW, class F>
__device__ __forceinline__ void with_wave(int w, F&& f) {
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  switch (w) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    default:
      if constexpr (NW == 8) {
        switch (w) {
          case 4: f(std::integral_constant<int, 4>{}); break;
          case 5: f(std::integral_constant<int, 5>{}); break;
          case 6: f(std::integral_constant<int, 6>{}); break;
          default: f(std::integral_constant<int, 7>{}); break;
        }
      }
      break;
  }
}

// s_waitcnt immediate (gfx9 encoding): vmcnt 0, expcnt and lgkmcnt unconstrained
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// lo(a) lo(b) + hi(a) hi(b) + c for bf16 pairs, fp32 accumulation
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;  // (1, 1) in bf16

// Score products Sc^T[key][query] = K Q^T with K = d.  At d = 16 the
// 16x16x16 form takes 4 bf16 per lane (k = 4g + i); at d = 32 the 16x16x32
// form takes 8 (k = 8g + i).
template <int DK>
struct ScoreOpT;
template <>
struct ScoreOpT<16> {
  using type = uint2;
};
template <>
struct ScoreOpT<32> {
  using type = u32x4;
};
template <int DK>
__device__ __forceinline__ f32x4 score_mfma(const typename ScoreOpT<DK>::type& a, const typename ScoreOpT<DK>::type& b) {
  if constexpr (DK == 16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b),
                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  } else {
    return mfma(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
  }
}

// Buffer resource over `rows` rows of `row_bytes` starting at row `row0` of
// `base`.  Buffer reads past the last row return 0 and writes past it are
// dropped by the hardware range check, which is how the ragged last chunk of
// a sequence is read and written.  The resource is uniform (scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t row0, int64_t rows,
                                                           int row_bytes) {
  char* p = const_cast<char*>(static_cast<const char*>(base)) + row0 * row_bytes;
  const int n = rows > 0 ? static_cast<int>(rows) * row_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0), n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, uint2 x) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.x, x.y}, r, off, 0, 0);
}

constexpr int OB_LD = DV + 8;  // bf16 row stride of a wave's output staging tile

// ------------------------------------------------------------ chunk sources
//
// Buffer resources over one chunk's rows of q, k, v (and the gate sums of the
// gated read).  Rows at or past the end read as zero.
struct ChunkSrc {
  __amdgpu_buffer_rsrc_t q, k, v;
  __amdgpu_buffer_rsrc_t g;   // per-token gate sums (gated read only)
  __amdgpu_buffer_rsrc_t gk;  // per-token key factors (gated read only)
};

template <int DK, int C>
__device__ __forceinline__ ChunkSrc chunk_src(const void* q, const void* k, const void* v, int64_t tok0,
                                              int64_t c0, int64_t T, const float* gb = nullptr,
                                              const float* gk = nullptr) {
  const int64_t n = (T - c0 < C) ? T - c0 : C;
  return ChunkSrc{rows_rsrc(q, tok0 + c0, n, 2 * DK), rows_rsrc(k, tok0 + c0, n, 2 * DK),
                  rows_rsrc(v, tok0 + c0, n, 2 * DV), rows_rsrc(gb, tok0 + c0, n, 4),
                  rows_rsrc(gk, tok0 + c0, n, 4)};
}

// ------------------------------------------------------------ LDS DMA and transposing reads

#define KATA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Swizzles of the LDS tiles against bank conflicts (measured on gfx950 with
// per-pattern read loops and SQ_LDS_BANK_CONFLICT):
//  - 128-byte rows (V, and the linear map's feature rows): the 32-byte piece
//    pair of row t is XORed with (t >> 1) & 3, i.e. 16-byte piece p is stored
//    at p ^ vswz(t).  A transposing read (4 rows x 32 bytes per 16 lanes) then
//    reaches 4 distinct pair positions and no bank twice: 4.5 cycles per read
//    per CU against 5.3 with the former (t >> 1) & 7 on 16-byte pieces; row
//    reads of 16 bytes per lane stay conflict-free.
//  - 32-byte rows (K and Q at d = 16, the key Gram matrix): the two 16-byte
//    pieces of row t are exchanged when ksw16(t) = (t >> 3) & 1 is set, so the
//    8-byte operand reads of 16 consecutive rows (score operands, query rows)
//    do not pair rows t and t + 8 on one bank: 4.8 cycles per read against 5.9.
__device__ __forceinline__ int vswz(int row) { return 2 * ((row >> 1) & 3); }
__device__ __forceinline__ int ksw16(int row) { return (row >> 3) & 1; }

__device__ __forceinline__ uint2 tr_read(const uint16_t* p) {
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint2, x);
}

// Per-lane element offsets of the transposing reads.  Lane (g, s) addresses
// row 4g + s/4 (+ 32 ks + 16 h), columns 4(s % 4)..+3 of the 16-column block;
// within a 32-row k-step the V swizzle vswz(row) reduces to 2 ((2g + s/8) & 3)
// and the K swizzle ksw16(row) to (g >> 1) & 1, so the offsets are lane
// constants and k-step / half are immediate offsets.
struct TrOffsets {
  int v[NDT - 1];  // V, per value tile
  int k;           // K
};

__device__ __forceinline__ TrOffsets tr_offsets(int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = 4 * g + (s >> 2);
  const int z = 2 * ((2 * g + (s >> 3)) & 3);
  TrOffsets o;
#pragma unroll
  for (int dt = 0; dt < NDT - 1; ++dt) {
    const int chunk = (2 * dt + ((s & 3) >> 1)) ^ z;
    o.v[dt] = row * DV + 8 * chunk + 4 * (s & 1);
  }
  o.k = row * 16 + 4 * ((s & 3) ^ (2 * ((g >> 1) & 1)));
  return o;
}

// operand of k-step ks: lane (g, r) gets column r of the block of tokens
// 32 ks + 4g + m and 32 ks + 16 + 4g + m (m = 0..3), the key order of a pair
// of 16x16 score accumulators
template <int LD>
__device__ __forceinline__ u32x4 tr_operand(const uint16_t* t, int off, int ks) {
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint2 x = tr_read(&t[off + (32 * ks + 16 * h) * LD]);
    out[2 * h] = x.x;
    out[2 * h + 1] = x.y;
  }
  return out;
}

// Span-sum update: wave W reduces feature tiles W and W + 4 over every k-step
// and the last tile (8) over the k-steps ks % 4 == W into acc8, so the waves
// carry equal work; the partial acc8 of the waves are added once per span.
// s_waitcnt immediate with vmcnt = n (gfx9 encoding), expcnt and lgkmcnt free
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Workgroup barrier that leaves vector-memory loads in flight: LDS reads and
// writes of this wave complete first (lgkmcnt), global loads and LDS DMA do
// not.  The memory clobber keeps the compiler from moving memory operations
// across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

}  // namespace
}  // namespace kata
