// Matrix-core (bf16 MFMA, fp32 accumulate) kernels of the chunked forward for
// d = 16 (D = 136), dv = 64, chunk 64 or 128 -- the KATA page, Sec. 4.1
// Eqs. 17-20: per chunk c of a span,
//   O_c = [phi_q(Q_c) S + ((Q_c K_c^T)^2 * M) V_c] / [phi_q(Q_c) z + ((Q_c K_c^T)^2 * M) 1 + eps]
//   S  += phi_k(K_c)^T V_c,   z += phi_k(K_c)^T 1
// with the incoming (S, z) of the span taken from the exclusive prefix over
// span sums (App. E.1 three-stage pipeline).
//
// Layout decisions (all private to the forward):
//  * Features.  The 136 products x_a x_b (a <= b) are placed on 160 feature
//    positions p = 32*ks + 8*g + i (ks: 32-wide MFMA k-step, g: lane group of
//    the 16x16x32 operand layout, i: slot).  Group g holds the pairs of group
//    0 shifted by 4g (mod 16) in both indices: every pair orbit under that
//    shift has 4 members, except the 4 orbits {(x, x+8), (x+4, x+12)} of 2.
//    A lane can then build its query-feature operand from its own query row
//    read rotated by 4g, with compile-time pair indices: phi(Q) never goes
//    through LDS.  Query features carry the off-diagonal factor 2, key
//    features none, so phi_q . phi_k = (q.k)^2.
//  * Denominators ride through the MFMAs: V gets a column of ones (tile 4 of
//    the value tiles), so P.1 and phi_q.z come out of the same products as
//    the numerators, and z is column 64 of the fp32 state.
//  * Tokens inside each 32-token k-step are stored in the order in which a
//    16x16 score accumulator hands them to the next product (the two 16-key
//    halves interleaved in groups of 4), so the squared scores feed P.V
//    straight from registers.
//  * The fp32 state S (feature tiles x 5 value tiles) lives in registers,
//    feature tiles split across the 4 waves; a bf16 copy in LDS is the
//    operand of the readout, which is split across waves by query tiles.
#include "common.h"
#include "kernels.h"
#include "plan_mfma.h"

namespace kata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int DK = 16;
constexpr int DV = 64;
constexpr int NDT = kMfmaValueTiles;     // 4 value tiles + the ones-column tile
constexpr int VROWS = 16 * NDT;          // 80
constexpr int DP = 160;                  // feature positions (5 k-steps of 32)
constexpr int NKS_F = DP / 32;           // feature k-steps of the readout
constexpr int NFT = kMfmaFeatureTiles;   // 9 feature tiles hold the 136 features
constexpr int SB_LD = DP + 8;            // LDS row stride of the bf16 state copy

// ------------------------------------------------------------ feature schedule

struct Schedule {
  int8_t a[40];
  int8_t b[40];
  bool pair2[40];  // orbit of size 2: only lane groups 0 and 1 carry it
};

constexpr Schedule make_schedule() {
  Schedule s{};
  bool used[16][16] = {};
  int n4 = 0, n2 = 32;
  for (int i = 0; i < 16; ++i) {
    for (int j = i; j < 16; ++j) {
      if (used[i][j]) continue;
      int size = 0;
      for (int g = 0; g < 4; ++g) {
        int x = (i + 4 * g) & 15, y = (j + 4 * g) & 15;
        if (x > y) { int t = x; x = y; y = t; }
        if (!used[x][y]) { used[x][y] = true; ++size; }
      }
      if (size == 4) {
        s.a[n4] = static_cast<int8_t>(i); s.b[n4] = static_cast<int8_t>(j); s.pair2[n4] = false; ++n4;
      } else {
        s.a[n2] = static_cast<int8_t>(i); s.b[n2] = static_cast<int8_t>(j); s.pair2[n2] = true; ++n2;
      }
    }
  }
  for (int e = 36; e < 40; ++e) { s.a[e] = -1; s.b[e] = -1; s.pair2[e] = false; }
  return s;
}

constexpr Schedule kSched = make_schedule();
__constant__ Schedule kSchedDev = make_schedule();

constexpr bool schedule_ok() {
  // 32 orbits of 4 and 4 of 2 cover the 136 pairs exactly once
  bool seen[16][16] = {};
  int n = 0;
  for (int e = 0; e < 36; ++e) {
    for (int g = 0; g < (kSched.pair2[e] ? 2 : 4); ++g) {
      int x = (kSched.a[e] + 4 * g) & 15, y = (kSched.b[e] + 4 * g) & 15;
      if (x > y) { int t = x; x = y; y = t; }
      if (seen[x][y]) return false;
      seen[x][y] = true;
      ++n;
    }
  }
  return n == 136;
}
static_assert(schedule_ok(), "feature schedule must cover every pair once");

// pair (a, b) on feature position p, or a = -1 for an empty position
__device__ __forceinline__ void pair_at(int p, int& a, int& b) {
  const int ks = p >> 5, o = p & 31, g = o >> 3, i = o & 7;
  const int e = 8 * ks + i;
  if (e >= 36 || (kSchedDev.pair2[e] && g >= 2)) { a = -1; b = -1; return; }
  a = (kSchedDev.a[e] + 4 * g) & 15;
  b = (kSchedDev.b[e] + 4 * g) & 15;
}

// ------------------------------------------------------------ small helpers

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

// position of the first of 4 consecutive tokens (group tg) inside a chunk:
// within each 32-token block, token groups 0..3 sit at 8a, groups 4..7 at
// 8(a-4)+4, matching the key order of a 16x16 accumulator pair.
__device__ __forceinline__ int group_pos(int tg) {
  const int a = tg & 7;
  return (tg >> 3) * 32 + ((a < 4) ? 8 * a : 8 * (a - 4) + 4);
}

// LDS tiles.  Row strides are padded so that the 16-byte operand reads of 16
// consecutive lanes (consecutive rows) land on distinct bank groups, and
// every row starts 16-byte aligned so the reads stay single b128 accesses.
constexpr int QF_LD = DK + 4;  // fp32 row stride of Q (80 B)
constexpr int KB_LD = DK + 8;  // bf16 row stride of K (48 B)

template <int C>
struct alignas(16) Smem {
  static constexpr int LDT = C + 8;       // bf16 row stride of Vt (C=128: 272 B)
  static constexpr int LDK = C + 4;       // fp32 row stride of Kt
  alignas(16) uint16_t Vt[DV * LDT];      // [value column][token position]
  alignas(16) float Kt[DK * LDK];         // [d][token position] fp32
};

template <int C>
struct alignas(16) SmemOut : Smem<C> {
  alignas(16) uint16_t Kb[C * KB_LD];     // [token][d] bf16 (score operand)
  alignas(16) float Qf[C * QF_LD];        // [token][d] fp32
  alignas(16) uint16_t Sb[VROWS * SB_LD]; // [value row][feature position] bf16 state copy
};

// ------------------------------------------------------------ chunk staging
//
// Global -> registers -> LDS for one chunk.  V: groups of 4 tokens x 8
// columns (16 B per token), written transposed; K and Q: one token row
// (32 B) per thread.  Tokens at or past T read as zero.
template <int C, bool WITH_Q>
struct Stage {
  static constexpr int NVG = (C / 4) * (DV / 8);
  uint4 v[4];
  uint4 kq[2];  // one K row (threads [0, C)) or one Q row (threads [C, 2C))

  __device__ __forceinline__ void load(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                       const uint16_t* __restrict__ vg, int64_t tok0, int64_t c0,
                                       int64_t T, int tid) {
    const bool full = c0 + C <= T;
    if (tid < NVG) {
      const int tg = tid % (C / 4), cg = tid / (C / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = c0 + 4 * tg + r;
        v[r] = (full || t < T) ? *reinterpret_cast<const uint4*>(vg + (tok0 + t) * DV + 8 * cg)
                               : make_uint4(0, 0, 0, 0);
      }
    }
    const int nrows = WITH_Q ? 2 * C : C;
    if (tid < nrows) {
      const bool is_q = WITH_Q && tid >= C;
      const int64_t t = c0 + (is_q ? tid - C : tid);
      const uint16_t* src = (is_q ? qg : kg) + (tok0 + t) * DK;
      if (full || t < T) {
        kq[0] = *reinterpret_cast<const uint4*>(src);
        kq[1] = *reinterpret_cast<const uint4*>(src + 8);
      } else {
        kq[0] = make_uint4(0, 0, 0, 0);
        kq[1] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  template <class S>
  __device__ __forceinline__ void store(S& sm, int tid) const {
    constexpr int LDT = Smem<C>::LDT, LDK = Smem<C>::LDK;
    if (tid < NVG) {
      const int tg = tid % (C / 4), cg = tid / (C / 4);
      const int pos = group_pos(tg);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t w0 = (x < 2) ? v[0].x : (x < 4) ? v[0].y : (x < 6) ? v[0].z : v[0].w;
        const uint32_t w1 = (x < 2) ? v[1].x : (x < 4) ? v[1].y : (x < 6) ? v[1].z : v[1].w;
        const uint32_t w2 = (x < 2) ? v[2].x : (x < 4) ? v[2].y : (x < 6) ? v[2].z : v[2].w;
        const uint32_t w3 = (x < 2) ? v[3].x : (x < 4) ? v[3].y : (x < 6) ? v[3].z : v[3].w;
        uint2 o;
        if (x & 1) {
          o.x = (w0 >> 16) | (w1 & 0xffff0000u);
          o.y = (w2 >> 16) | (w3 & 0xffff0000u);
        } else {
          o.x = (w0 & 0xffffu) | (w1 << 16);
          o.y = (w2 & 0xffffu) | (w3 << 16);
        }
        *reinterpret_cast<uint2*>(&sm.Vt[(8 * cg + x) * LDT + pos]) = o;
      }
    }
    if (tid < C) {
      // K row: fp32 transposed copy (key features) and, with Q, a bf16 row copy (scores)
      const int t = tid;
      const int pos = group_pos(t >> 2) + (t & 3);
      const uint32_t w[8] = {kq[0].x, kq[0].y, kq[0].z, kq[0].w, kq[1].x, kq[1].y, kq[1].z, kq[1].w};
#pragma unroll
      for (int x = 0; x < DK; ++x) {
        sm.Kt[x * LDK + pos] = (x & 1) ? hi_bf16(w[x >> 1]) : lo_bf16(w[x >> 1]);
      }
      if constexpr (WITH_Q) {
        *reinterpret_cast<uint4*>(&sm.Kb[t * KB_LD]) = kq[0];
        *reinterpret_cast<uint4*>(&sm.Kb[t * KB_LD + 8]) = kq[1];
      }
    } else if (WITH_Q && tid < 2 * C) {
      if constexpr (WITH_Q) {
        const int t = tid - C;
        const uint32_t w[8] = {kq[0].x, kq[0].y, kq[0].z, kq[0].w, kq[1].x, kq[1].y, kq[1].z, kq[1].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float4 f;
          f.x = lo_bf16(w[2 * c]);
          f.y = hi_bf16(w[2 * c]);
          f.z = lo_bf16(w[2 * c + 1]);
          f.w = hi_bf16(w[2 * c + 1]);
          *reinterpret_cast<float4*>(&sm.Qf[t * QF_LD + 4 * c]) = f;
        }
      }
    }
  }
};

// The ones column of [V | 1 | 0]: value tile 4 holds 1.0 in its first column
// (lane r == 0 of every lane group) and zeros elsewhere, for every token slot.
__device__ __forceinline__ u32x4 ones_frag(int r) {
  const uint32_t one2 = 0x3f803f80u;  // two bf16 1.0
  return (r == 0) ? u32x4{one2, one2, one2, one2} : u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------ state update
//
// acc[m][dt] += phi_k(K_c)^T [V_c | 1 | 0] for the feature tiles ft = w + 4m
// this wave owns.  The key-feature operand (position 16 ft + r, 8 token
// slots) is built from two fp32 rows of K^T.
struct KeyPairs {
  int a[3];
  int b[3];
};

__device__ __forceinline__ KeyPairs key_pairs(int w, int r) {
  KeyPairs kp;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int ft = w + 4 * m;
    int a = -1, b = -1;
    if (ft < NFT) pair_at(16 * ft + r, a, b);
    kp.a[m] = a;
    kp.b[m] = b;
  }
  return kp;
}

template <int C, class S>
__device__ __forceinline__ void state_update(f32x4 (&acc)[3][NDT], const S& sm, int w, int lane,
                                             const KeyPairs& kp, const u32x4& ones) {
  constexpr int LDT = Smem<C>::LDT, LDK = Smem<C>::LDK;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int ks = 0; ks < C / 32; ++ks) {
    u32x4 bv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) {
      bv[dt] = *reinterpret_cast<const u32x4*>(&sm.Vt[(16 * dt + r) * LDT + 32 * ks + 8 * g]);
    }
    bv[NDT - 1] = ones;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      if (w + 4 * m >= NFT) continue;  // uniform per wave
      u32x4 af = {0u, 0u, 0u, 0u};
      if (kp.a[m] >= 0) {
        const float* ra = &sm.Kt[kp.a[m] * LDK + 32 * ks + 8 * g];
        const float* rb = &sm.Kt[kp.b[m] * LDK + 32 * ks + 8 * g];
        const float4 a0 = *reinterpret_cast<const float4*>(ra);
        const float4 a1 = *reinterpret_cast<const float4*>(ra + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(rb);
        const float4 b1 = *reinterpret_cast<const float4*>(rb + 4);
        af.x = pack2(a0.x * b0.x, a0.y * b0.y);
        af.y = pack2(a0.z * b0.z, a0.w * b0.w);
        af.z = pack2(a1.x * b1.x, a1.y * b1.y);
        af.w = pack2(a1.z * b1.z, a1.w * b1.w);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[m][dt] = mfma(af, bv[dt], acc[m][dt]);
    }
  }
}

// fp32 state tiles <-> workspace.  Value tiles 0..3 in tile-native order
// ((ft*4 + dt)*64 + lane)*4 + j; the ones-column tile only carries z in its
// column 0 (lanes r == 0), stored as 16 floats per feature tile.
constexpr int kZOffset = NFT * (NDT - 1) * 256;

__device__ __forceinline__ void load_state(f32x4 (&acc)[3][NDT], const float* __restrict__ P,
                                           int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int ft = w + 4 * m;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (P == nullptr || ft >= NFT) continue;
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) {
      const float4 x = *reinterpret_cast<const float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4);
      acc[m][dt] = f32x4{x.x, x.y, x.z, x.w};
    }
    if (r == 0) {
      const float4 x = *reinterpret_cast<const float4*>(P + kZOffset + ft * 16 + 4 * g);
      acc[m][NDT - 1] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
}

__device__ __forceinline__ void store_state(const f32x4 (&acc)[3][NDT], float* __restrict__ P,
                                            int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int ft = w + 4 * m;
    if (ft >= NFT) continue;
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) {
      *reinterpret_cast<float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4) =
          make_float4(acc[m][dt][0], acc[m][dt][1], acc[m][dt][2], acc[m][dt][3]);
    }
    if (r == 0) {
      *reinterpret_cast<float4*>(P + kZOffset + ft * 16 + 4 * g) =
          make_float4(acc[m][NDT - 1][0], acc[m][NDT - 1][1], acc[m][NDT - 1][2],
                      acc[m][NDT - 1][3]);
    }
  }
}

// bf16 copy of the owned state tiles into Sb[value row][feature position]
template <class S>
__device__ __forceinline__ void write_sb(S& sm, const f32x4 (&acc)[3][NDT], int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int ft = w + 4 * m;
    if (ft >= NFT) continue;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 o;
      o.x = pack2(acc[m][dt][0], acc[m][dt][1]);
      o.y = pack2(acc[m][dt][2], acc[m][dt][3]);
      *reinterpret_cast<uint2*>(&sm.Sb[(16 * dt + r) * SB_LD + 16 * ft + 4 * g]) = o;
    }
  }
}

// ------------------------------------------------------------ span sums

template <int C>
__global__ __launch_bounds__(kThreads) void span_state_mfma_kernel(MfmaArgs a) {
  __shared__ Smem<C> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t nsp_work = a.n_spans - 1;  // the last span's sum is never read
  const int64_t bh = blockIdx.x / nsp_work;
  const int64_t sp = blockIdx.x - bh * nsp_work;
  const int64_t tok0 = bh * a.T;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);

  const KeyPairs kp = key_pairs(w, lane & 15);
  const u32x4 ones = ones_frag(lane & 15);
  f32x4 acc[3][NDT];
  load_state(acc, nullptr, w, lane);

  // two register stages: chunk i+2 is in flight while chunk i is consumed
  const int64_t first = sp * a.G * C;
  int64_t end = first + a.G * C;
  if (end > a.T) end = a.T;
  Stage<C, false> st0, st1;
  st0.load(nullptr, kg, vg, tok0, first, a.T, tid);
  if (first + C < end) st1.load(nullptr, kg, vg, tok0, first + C, a.T, tid);
  for (int64_t c0 = first; c0 < end; c0 += 2 * C) {
    __syncthreads();
    st0.store(sm, tid);
    if (c0 + 2 * C < end) st0.load(nullptr, kg, vg, tok0, c0 + 2 * C, a.T, tid);
    __syncthreads();
    state_update<C>(acc, sm, w, lane, kp, ones);
    if (c0 + C >= end) break;
    __syncthreads();
    st1.store(sm, tid);
    if (c0 + 3 * C < end) st1.load(nullptr, kg, vg, tok0, c0 + 3 * C, a.T, tid);
    __syncthreads();
    state_update<C>(acc, sm, w, lane, kp, ones);
  }
  store_state(acc, a.ws + (bh * a.n_spans + sp) * kMfmaStateFloats, w, lane);
}

// ------------------------------------------------------------ readout

// query tiles of each wave, balanced for the causal work: {slot0, slot1}
template <int C>
__device__ __forceinline__ int query_tile(int w, int slot) {
  if constexpr (C == 128) {
    constexpr int t[4][2] = {{0, 1}, {2, 7}, {3, 6}, {4, 5}};
    return t[w][slot];
  } else {
    return slot == 0 ? w : -1;
  }
}

template <int C>
__global__ __launch_bounds__(kThreads, 2) void readout_mfma_kernel(MfmaArgs a) {
  __shared__ SmemOut<C> sm;
  constexpr int LDT = Smem<C>::LDT;
  constexpr int NSLOT = (C == 128) ? 2 : 1;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t bh = blockIdx.x / a.n_spans;
  const int64_t sp = blockIdx.x - bh * a.n_spans;
  const int64_t tok0 = bh * a.T;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);
  uint16_t* og = static_cast<uint16_t*>(a.out);

  // feature positions 144..159 hold no feature: keep their state copy zero
  for (int e = tid; e < VROWS * 16; e += kThreads) sm.Sb[(e >> 4) * SB_LD + 144 + (e & 15)] = 0;
  const KeyPairs kp = key_pairs(w, r);
  const u32x4 ones = ones_frag(r);
  f32x4 acc[3][NDT];
  load_state(acc, a.n_spans > 1 ? a.ws + (bh * a.n_spans + sp) * kMfmaStateFloats : nullptr, w,
             lane);
  write_sb(sm, acc, w, lane);

  int qt[NSLOT];
#pragma unroll
  for (int slot = 0; slot < NSLOT; ++slot) qt[slot] = query_tile<C>(w, slot);
  const int qt_max = qt[NSLOT - 1] > qt[0] ? qt[NSLOT - 1] : qt[0];
  const float keep2 = (g < 2) ? 1.0f : 0.0f;

  Stage<C, true> st;
  int64_t c0 = sp * a.G * C;
  st.load(qg, kg, vg, tok0, c0, a.T, tid);
  for (int64_t gi = 0; gi < a.G; ++gi, c0 += C) {
    if (c0 >= a.T) break;
    __syncthreads();  // previous chunk: all reads of the staged tiles done, Sb written
    st.store(sm, tid);
    if (gi + 1 < a.G && c0 + C < a.T) st.load(qg, kg, vg, tok0, c0 + C, a.T, tid);
    __syncthreads();

    // ---- readout of this chunk's queries (state = prefix before the chunk).
    // Computed transposed, O^T = [S|z]^T phi_q(Q)^T + [V|1]^T P^T, so a lane
    // ends up holding 4 consecutive value columns of one query.
    f32x4 o[NSLOT][NDT];
    float qr[NSLOT][DK];  // this lane's query row (query 16 qt + r), rotated by 4g
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[slot][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 x =
            *reinterpret_cast<const float4*>(&sm.Qf[(16 * qt[slot] + r) * QF_LD + 4 * ((c + g) & 3)]);
        qr[slot][4 * c + 0] = x.x;
        qr[slot][4 * c + 1] = x.y;
        qr[slot][4 * c + 2] = x.z;
        qr[slot][4 * c + 3] = x.w;
      }
    }
    // inter-chunk term
#pragma unroll
    for (int ks = 0; ks < NKS_F; ++ks) {
      u32x4 bs[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bs[dt] = *reinterpret_cast<const u32x4*>(&sm.Sb[(16 * dt + r) * SB_LD + 32 * ks + 8 * g]);
      }
#pragma unroll
      for (int slot = 0; slot < NSLOT; ++slot) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = 8 * ks + i;
          if (e >= 36) {
            f[i] = 0.f;
          } else {
            const int pa = kSched.a[e], pb = kSched.b[e];
            const float x = (pa == pb) ? qr[slot][pa] * qr[slot][pa]
                                       : (2.0f * qr[slot][pa]) * qr[slot][pb];
            f[i] = kSched.pair2[e] ? x * keep2 : x;
          }
        }
        const u32x4 qfeat = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[slot][dt] = mfma(bs[dt], qfeat, o[slot][dt]);
      }
    }
    // intra-chunk term: squared causal scores
    u32x4 qf[NSLOT];
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      qf[slot] = u32x4{0u, 0u, 0u, 0u};
      if (g < 2) {
        const float* qrow = &sm.Qf[(16 * qt[slot] + r) * QF_LD + 8 * g];
        const float4 x0 = *reinterpret_cast<const float4*>(qrow);
        const float4 x1 = *reinterpret_cast<const float4*>(qrow + 4);
        qf[slot] = u32x4{pack2(x0.x, x0.y), pack2(x0.z, x0.w), pack2(x1.x, x1.y), pack2(x1.z, x1.w)};
      }
    }
#pragma unroll
    for (int s = 0; s < C / 32; ++s) {
      if (2 * s > qt_max) break;
      u32x4 kf[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        kf[h] = u32x4{0u, 0u, 0u, 0u};
        if (g < 2) kf[h] = *reinterpret_cast<const u32x4*>(&sm.Kb[(16 * (2 * s + h) + r) * KB_LD + 8 * g]);
      }
      u32x4 bv[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) {
        bv[dt] = *reinterpret_cast<const u32x4*>(&sm.Vt[(16 * dt + r) * LDT + 32 * s + 8 * g]);
      }
      bv[NDT - 1] = ones;
#pragma unroll
      for (int slot = 0; slot < NSLOT; ++slot) {
        if (2 * s > qt[slot]) continue;  // uniform per wave
        float p[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kt = 2 * s + h;
          const f32x4 sc = mfma(kf[h], qf[slot], f32x4{0.f, 0.f, 0.f, 0.f});  // [key 4g+j][query r]
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = sc[j] * sc[j];
            p[h][j] = (kt > qt[slot] || (kt == qt[slot] && 4 * g + j > r)) ? 0.f : x;
          }
        }
        const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                          pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[slot][dt] = mfma(bv[dt], pf, o[slot][dt]);
      }
    }
    // normalise and store: lane r of group 0 holds the denominator of query r
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      const float den = __shfl(o[slot][NDT - 1][0], r);
      const float inv = __builtin_amdgcn_rcpf(den + a.eps);
      const int64_t t = c0 + 16 * qt[slot] + r;
      if (t < a.T) {
        uint16_t* dst = og + (tok0 + t) * DV + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt) {
          uint2 ob;
          ob.x = pack2(o[slot][dt][0] * inv, o[slot][dt][1] * inv);
          ob.y = pack2(o[slot][dt][2] * inv, o[slot][dt][3] * inv);
          *reinterpret_cast<uint2*>(dst + 16 * dt) = ob;
        }
      }
    }

    // ---- carry the state across the chunk
    if (gi + 1 < a.G && c0 + C < a.T) {
      state_update<C>(acc, sm, w, lane, kp, ones);
      __syncthreads();  // every wave done reading Sb for this chunk
      write_sb(sm, acc, w, lane);
    }
  }
}

}  // namespace

hipError_t launch_span_state_mfma(const MfmaArgs& a, hipStream_t stream) {
  if (a.n_spans < 2) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.BH * (a.n_spans - 1)));
  switch (a.chunk) {
    case 64: span_state_mfma_kernel<64><<<grid, kThreads, 0, stream>>>(a); break;
    case 128: span_state_mfma_kernel<128><<<grid, kThreads, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_readout_mfma(const MfmaArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.BH * a.n_spans));
  switch (a.chunk) {
    case 64: readout_mfma_kernel<64><<<grid, kThreads, 0, stream>>>(a); break;
    case 128: readout_mfma_kernel<128><<<grid, kThreads, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kata
