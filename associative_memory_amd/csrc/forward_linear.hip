// The chunked read with linear (D = d = 64) features on the matrix cores:
// the KATA-Orthant and KATA-Lorentz cone maps (normalised read) and the
// identity map psi(x) = x (first-order read, no denominator); see the kernel
// comment below.
#include "mfma_common.h"

namespace kata {
namespace {

// ------------------------------------------------------------ linear features
//
// The chunked read with a linear feature psi (D = d = 64) through the same
// three stages as the PSD map (the KATA page, Sec. 4.1 Eqs. 17-20 with the
// unsquared score psi(q) . psi(k)): KATA-Orthant and KATA-Lorentz (App. F.4)
// read o = N / (D + eps); the identity map of the page's first-order tables
// (Sec. 4.2, Tables 10-11) reads N alone, its scores being signed.  Per chunk
// of C tokens (32, 64 or 128) the raw K and Q rows pass through registers,
// where psi is applied in fp32 (orthant: ReLU(x) + shift per coordinate;
// Lorentz: (y, |y| (1 + s^2)), |y| summed over the 4 lanes that hold a row;
// identity: the bf16 rows as they are), and land in LDS as bf16 rows in the V
// layout (16-byte pieces swizzled by vswz(row)); V arrives by DMA into
// two buffers.  The fp32 state [S | z] (64 features x 65; S alone for the
// identity map) is one feature tile per wave; psi(K)^T and [V | 1] operands
// of its update both come from transposing LDS reads.  The readout computes
// O^T = [S|z]^T psi(Q)^T + [V|1]^T P^T, P = (psi(K) psi(Q)^T)^T masked, with
// the query tiles split over the 4 waves: one each at C = 64, two at C = 128
// (tiles W and 7 - W, equal causal work), and at C = 32 two waves per query
// tile splitting the value tiles (both carrying the denominator tile).
constexpr int LSB = DV + 8;  // bf16 row stride of the state copy [value row][feature]

template <int FEAT>
constexpr bool kNormalised = FEAT != kLinFeatIdentity;

// accumulator value tiles of the state: four of S, plus z for the normalised maps
template <int FEAT>
constexpr int lin_state_tiles() { return kNormalised<FEAT> ? NDT : NDT - 1; }

template <int C>
struct alignas(16) LinRows {
  alignas(16) uint16_t r[C * 64];  // [token][64], 16-byte pieces swizzled by vswz
};

// Quarter rows (16 dimensions) of K and of Q per thread: rows tid / 4 + 64 u
// (u < NR), dimensions 16 (tid % 4) .. +15.  Rows past the sequence read as
// zero and are written as zero features.
template <int FEAT, bool WITH_Q, int C>
struct LinStage {
  static constexpr int NR = C >= 64 ? C / 64 : 1;  // rows per thread
  static constexpr int NTH = 4 * C / NR;           // threads holding rows
  u32x4 k[NR][2];
  u32x4 q[NR][2];

  __device__ __forceinline__ void load(const ChunkSrc& src, int tid) {
    if (tid >= NTH) return;  // uniform per wave
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int off = ((tid >> 2) + 64 * u) * 128 + 32 * (tid & 3);
      k[u][0] = __builtin_amdgcn_raw_buffer_load_b128(src.k, off, 0, 0);
      k[u][1] = __builtin_amdgcn_raw_buffer_load_b128(src.k, off + 16, 0, 0);
      if constexpr (WITH_Q) {
        q[u][0] = __builtin_amdgcn_raw_buffer_load_b128(src.q, off, 0, 0);
        q[u][1] = __builtin_amdgcn_raw_buffer_load_b128(src.q, off + 16, 0, 0);
      }
    }
  }

  // psi of one quarter row, written to its swizzled place
  static __device__ __forceinline__ void put(uint16_t* rows, const u32x4 (&x)[2], int row, int qq, bool valid,
                                             float shift) {
    if constexpr (FEAT == kLinFeatIdentity) {
      // psi(x) = x: the bf16 row as loaded (zero past the sequence)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = (2 * qq + h) ^ vswz(row);
        *reinterpret_cast<u32x4*>(&rows[row * 64 + 8 * c]) = x[h];
      }
      return;
    }
    float f[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * h + 2 * i] = lo_bf16(x[h][i]);
        f[8 * h + 2 * i + 1] = hi_bf16(x[h][i]);
      }
    }
    if constexpr (FEAT == kLinFeatOrthant) {
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = __builtin_fmaxf(f[i], 0.f) + shift;
    } else {
      // |y|^2 over dimensions 0..62: the last quarter leaves out its last entry (s)
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 15; ++i) ss = __builtin_fmaf(f[i], f[i], ss);
      if (qq != 3) ss = __builtin_fmaf(f[15], f[15], ss);
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if (qq == 3) f[15] = __builtin_sqrtf(ss) * __builtin_fmaf(f[15], f[15], 1.f);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (2 * qq + h) ^ vswz(row);
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = valid ? pack2(f[8 * h + 2 * i], f[8 * h + 2 * i + 1]) : 0u;
      *reinterpret_cast<u32x4*>(&rows[row * 64 + 8 * c]) = y;
    }
  }

  __device__ __forceinline__ void store(LinRows<C>& kr, LinRows<C>* qr, int tid, int64_t valid_rows,
                                        float shift) const {
    if (tid >= NTH) return;  // uniform per wave
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int row = (tid >> 2) + 64 * u;
      const bool valid = row < valid_rows;
      put(kr.r, k[u], row, tid & 3, valid, shift);
      if constexpr (WITH_Q) put(qr->r, q[u], row, tid & 3, valid, shift);
    }
  }
};

// 16-byte row operand: row t, dimensions 32 kf + 8 g .. +7
__device__ __forceinline__ u32x4 lin_row_op(const uint16_t* rows, int t, int kf, int g) {
  return *reinterpret_cast<const u32x4*>(&rows[t * 64 + 8 * ((4 * kf + g) ^ vswz(t))]);
}

// wave W's share of a chunk's V transfer (pieces of 8 rows)
template <int W, int C>
__device__ __forceinline__ void dma_lin_v(LinRows<C>& b, const ChunkSrc& src, int lane) {
#pragma unroll
  for (int j = W; j < C / 8; j += 4) {
    const int t = 8 * j + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.r[8 * j * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
}

// acc[i] += psi(K)^T [V | 1] for feature tile W over the chunk
template <int FEAT, int W, int C>
__device__ __forceinline__ void lin_state_update(f32x4 (&acc)[NDT], const LinRows<C>& kr, const LinRows<C>& vb,
                                                 const TrOffsets& to, const u32x4& bones) {
  constexpr int NST = lin_state_tiles<FEAT>();
#pragma unroll
  for (int s = 0; s < C / 32; ++s) {
    const u32x4 ak = tr_operand<64>(kr.r, to.v[W], s);
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const u32x4 bv = i < NDT - 1 ? tr_operand<DV>(vb.r, to.v[i], s) : bones;
      acc[i] = mfma(ak, bv, acc[i]);
    }
  }
}

// workspace layout of a span state: [feature tile][value tile][lane] f32x4
template <int FEAT>
__device__ __forceinline__ int lin_state_off(int W, int i, int lane) {
  return ((W * lin_state_tiles<FEAT>() + i) * 64 + lane) * 4;
}

template <int FEAT>
constexpr int64_t lin_state_floats() { return int64_t(4) * lin_state_tiles<FEAT>() * 256; }
static_assert(lin_state_floats<kLinFeatOrthant>() == kLinStateFloats, "workspace sizing");

template <int FEAT, int C>
__device__ __forceinline__ void lin_span_body(const LinArgs& a) {
  __shared__ LinRows<C> kr;
  __shared__ LinRows<C> v0;
  __shared__ LinRows<C> v1;
  __shared__ alignas(16) uint16_t ones[128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nsp = a.n_spans - 1;  // the last span's sum is not needed
  const int64_t bh = blockIdx.x / nsp;
  const int64_t sp = blockIdx.x - bh * nsp;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * C;
  const int64_t end = (a.T < first + a.G * C) ? a.T : first + a.G * C;
  if (tid < 128) ones[tid] = tid < 64 ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);

  with_wave<4>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int NST = lin_state_tiles<FEAT>();
    const int g = lane >> 4, r = lane & 15;
    const TrOffsets to = tr_offsets(lane);
    f32x4 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto src = [&](int64_t c0) { return chunk_src<64, C>(nullptr, a.k, a.v, tok0, c0, end); };
    LinStage<FEAT, false, C> st;
    st.load(src(first), tid);
    dma_lin_v<W, C>(v0, src(first), lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    st.store(kr, nullptr, tid, end - first, a.shift);
    __syncthreads();
    const u32x4 bones = *reinterpret_cast<const u32x4*>(&ones[(r > 0 ? 64 : 0) + 8 * g]);
    // chunk loop, unrolled over the two V buffers
    for (int64_t c0 = first; c0 < end; c0 += 2 * C) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * C;
        if (c >= end) break;
        LinRows<C>& cur = u == 0 ? v0 : v1;
        LinRows<C>& nxt = u == 0 ? v1 : v0;
        const bool more = c + C < end;
        if (more) {
          st.load(src(c + C), tid);
          dma_lin_v<W, C>(nxt, src(c + C), lane);
        }
        lin_state_update<FEAT, W, C>(acc, kr, cur, to, bones);
        barrier_lds();
        if (more) {
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          st.store(kr, nullptr, tid, end - (c + C), a.shift);
        }
        barrier_lds();
      }
    }
    float* dst = a.ws + (bh * a.n_spans + sp) * lin_state_floats<FEAT>();
#pragma unroll
    for (int i = 0; i < NST; ++i) *reinterpret_cast<f32x4*>(&dst[lin_state_off<FEAT>(W, i, lane)]) = acc[i];
  });
}

template <int FEAT, int C>
__global__ __launch_bounds__(256, 2) void lin_span_kernel(LinArgs a) {
  lin_span_body<FEAT, C>(a);
}

// the bf16 state copy [value row][feature] for the readout: rows 0..63 are
// S^T, row 64 is z (normalised maps), row 65 stays zero
template <int FEAT, int W>
__device__ __forceinline__ void lin_write_sb(uint16_t* sb, const f32x4 (&acc)[NDT], int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < NDT - 1; ++i) {
    uint2 x;
    x.x = pack2(acc[i][0], acc[i][1]);
    x.y = pack2(acc[i][2], acc[i][3]);
    *reinterpret_cast<uint2*>(&sb[(16 * i + r) * LSB + 16 * W + 4 * g]) = x;
  }
  if (kNormalised<FEAT> && r == 0) {
    uint2 x;
    x.x = pack2(acc[NDT - 1][0], acc[NDT - 1][1]);
    x.y = pack2(acc[NDT - 1][2], acc[NDT - 1][3]);
    *reinterpret_cast<uint2*>(&sb[DV * LSB + 16 * W + 4 * g]) = x;
  }
}

// the readout split of a chunk of C tokens over the 4 waves
template <int FEAT, int C>
struct LinSplit {
  static constexpr int NSLOT = C == 128 ? 2 : 1;  // query tiles per wave
  static constexpr bool SPLIT_V = C == 32;        // two waves per query tile
  // value tiles a wave reads out: all (with the denominator tile for the
  // normalised maps), or half of them with the denominator tile
  static constexpr int NO = SPLIT_V ? (kNormalised<FEAT> ? 3 : 2) : (kNormalised<FEAT> ? NDT : NDT - 1);
  // whole 16 x 64 output tiles staged through LDS as 16-byte stores (not at
  // C = 128, where the staging tiles would exceed the LDS of two workgroups)
  static constexpr bool STAGE_OUT = !SPLIT_V && C != 128;
  static __device__ __forceinline__ constexpr int qtile(int W, int slot) {
    return C == 128 ? (slot == 0 ? W : 7 - W) : (C == 64 ? W : (W & 1));
  }
  static __device__ __forceinline__ constexpr int vtile(int W, int i) {
    return SPLIT_V ? (i < 2 ? 2 * (W >> 1) + i : NDT - 1) : i;
  }
};

template <int FEAT, int C>
__device__ __forceinline__ void lin_readout_body(const LinArgs& a) {
  using SP = LinSplit<FEAT, C>;
  constexpr int NSLOT = SP::NSLOT, NO = SP::NO;
  __shared__ LinRows<C> kr;
  __shared__ LinRows<C> qr;
  __shared__ LinRows<C> v0;
  __shared__ LinRows<C> v1;
  __shared__ alignas(16) uint16_t sb[(DV + 2) * LSB];
  __shared__ alignas(16) uint16_t ones[128];
  __shared__ alignas(16) uint16_t Ob[SP::STAGE_OUT ? 4 : 1][SP::STAGE_OUT ? 16 * OB_LD : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / a.n_spans;
  const int64_t sp = blockIdx.x - bh * a.n_spans;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * C;
  const int64_t end = (a.T < first + a.G * C) ? a.T : first + a.G * C;
  if (tid < 128) ones[tid] = tid < 64 ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);
  if (tid < LSB / 8) *reinterpret_cast<uint4*>(&sb[(DV + 1) * LSB + 8 * tid]) = make_uint4(0, 0, 0, 0);

  with_wave<4>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int NST = lin_state_tiles<FEAT>();
    const int g = lane >> 4, r = lane & 15;
    bool keep[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) keep[j] = 4 * g + j <= r;
    const TrOffsets to = tr_offsets(lane);
    f32x4 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.n_spans > 1) {
      const float* P = a.ws + (bh * a.n_spans + sp) * lin_state_floats<FEAT>();
#pragma unroll
      for (int i = 0; i < NST; ++i) acc[i] = *reinterpret_cast<const f32x4*>(&P[lin_state_off<FEAT>(W, i, lane)]);
    }
    auto src = [&](int64_t c0) { return chunk_src<64, C>(a.q, a.k, a.v, tok0, c0, end); };
    LinStage<FEAT, true, C> st;
    st.load(src(first), tid);
    dma_lin_v<W, C>(v0, src(first), lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    lin_write_sb<FEAT, W>(sb, acc, lane);
    st.store(kr, &qr, tid, end - first, a.shift);
    __syncthreads();
    const u32x4 bones = *reinterpret_cast<const u32x4*>(&ones[(r > 0 ? 64 : 0) + 8 * g]);
    for (int64_t c0 = first; c0 < end; c0 += 2 * C) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * C;
        if (c >= end) break;
        LinRows<C>& cur = u == 0 ? v0 : v1;
        LinRows<C>& nxt = u == 0 ? v1 : v0;
        const bool more = c + C < end;
        // the query tiles' operands, then the next chunk's loads
        u32x4 qop[NSLOT][2];
#pragma unroll
        for (int slot = 0; slot < NSLOT; ++slot) {
#pragma unroll
          for (int kf = 0; kf < 2; ++kf) qop[slot][kf] = lin_row_op(qr.r, 16 * SP::qtile(W, slot) + r, kf, g);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          st.load(src(c + C), tid);
          dma_lin_v<W, C>(nxt, src(c + C), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        // inter-chunk term: [S|z]^T psi(Q)^T
        f32x4 o[NSLOT][NO];
#pragma unroll
        for (int i = 0; i < NO; ++i) {
#pragma unroll
          for (int slot = 0; slot < NSLOT; ++slot) o[slot][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kf = 0; kf < 2; ++kf) {
            const u32x4 as = *reinterpret_cast<const u32x4*>(&sb[vrow(SP::vtile(W, i), r) * LSB + 32 * kf + 8 * g]);
#pragma unroll
            for (int slot = 0; slot < NSLOT; ++slot) o[slot][i] = mfma(as, qop[slot][kf], o[slot][i]);
          }
        }
        // intra-chunk term over the key steps up to the diagonal, and the
        // state update over the whole chunk
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          u32x4 bv[NDT];
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) bv[i] = tr_operand<DV>(cur.r, to.v[i], s);
          bv[NDT - 1] = bones;
#pragma unroll
          for (int slot = 0; slot < NSLOT; ++slot) {
            const int qt = SP::qtile(W, slot);
            if (2 * s > qt) continue;  // compile-time per wave
            float p[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int kt = 2 * s + h;
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = 0.f;
              if (kt > qt) continue;
              f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kf = 0; kf < 2; ++kf) sc = mfma(lin_row_op(kr.r, 16 * kt + r, kf, g), qop[slot][kf], sc);
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = (kt < qt || keep[j]) ? sc[j] : 0.f;
            }
            const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                              pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
            for (int i = 0; i < NO; ++i) o[slot][i] = mfma(bv[SP::vtile(W, i)], pf, o[slot][i]);
          }
          const u32x4 ak = tr_operand<64>(kr.r, to.v[W], s);
#pragma unroll
          for (int i = 0; i < NST; ++i) acc[i] = mfma(ak, bv[i], acc[i]);
        }
        // normalise (cone maps) and store
        const int64_t n = end - c < C ? end - c : C;
        const __amdgpu_buffer_rsrc_t dst = rows_rsrc(a.out, tok0 + c, n, 2 * DV);
#pragma unroll
        for (int slot = 0; slot < NSLOT; ++slot) {
          const int qt = SP::qtile(W, slot);
          float inv = 1.f;
          if constexpr (kNormalised<FEAT>) {
            const float den = __shfl(o[slot][NO - 1][0], r);
            inv = __builtin_amdgcn_rcpf(den + a.eps);
          }
          constexpr int NVAL = kNormalised<FEAT> ? NO - 1 : NO;  // value tiles among the outputs
          if constexpr (SP::STAGE_OUT) {
            uint16_t* ob = Ob[W];
#pragma unroll
            for (int i = 0; i < NVAL; ++i) {
              uint2 x;
              x.x = pack2(o[slot][i][0] * inv, o[slot][i][1] * inv);
              x.y = pack2(o[slot][i][2] * inv, o[slot][i][3] * inv);
              *reinterpret_cast<uint2*>(&ob[r * OB_LD + 16 * SP::vtile(W, i) + 4 * g]) = x;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int row = 8 * h + (lane >> 3);
              const uint4 x = *reinterpret_cast<const uint4*>(&ob[row * OB_LD + 8 * (lane & 7)]);
              __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, dst,
                                                     (16 * qt + row) * (2 * DV) + 16 * (lane & 7), 0, 0);
            }
          } else {
            const int row = 16 * qt + r;
#pragma unroll
            for (int i = 0; i < NVAL; ++i) {
              uint2 x;
              x.x = pack2(o[slot][i][0] * inv, o[slot][i][1] * inv);
              x.y = pack2(o[slot][i][2] * inv, o[slot][i][3] * inv);
              buf_store8(dst, row * (2 * DV) + 2 * (16 * SP::vtile(W, i) + 4 * g), x);
            }
          }
        }
        barrier_lds();
        if (more) {
          lin_write_sb<FEAT, W>(sb, acc, lane);
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          st.store(kr, &qr, tid, end - (c + C), a.shift);
        }
        barrier_lds();
      }
    }
  });
}

template <int FEAT, int C>
__global__ __launch_bounds__(256, 2) void lin_readout_kernel(LinArgs a) {
  lin_readout_body<FEAT, C>(a);
}

template <int FEAT>
hipError_t launch_span_feat(const LinArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.chunk) {
    case 32: lin_span_kernel<FEAT, 32><<<grid, 256, 0, stream>>>(a); break;
    case 64: lin_span_kernel<FEAT, 64><<<grid, 256, 0, stream>>>(a); break;
    case 128: lin_span_kernel<FEAT, 128><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FEAT>
hipError_t launch_readout_feat(const LinArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.chunk) {
    case 32: lin_readout_kernel<FEAT, 32><<<grid, 256, 0, stream>>>(a); break;
    case 64: lin_readout_kernel<FEAT, 64><<<grid, 256, 0, stream>>>(a); break;
    case 128: lin_readout_kernel<FEAT, 128><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t linear_state_floats(int feature) {
  return feature == kLinFeatIdentity ? lin_state_floats<kLinFeatIdentity>() : lin_state_floats<kLinFeatOrthant>();
}

hipError_t launch_linear_span_state(const LinArgs& a, hipStream_t stream) {
  if (a.n_spans < 2) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.BH * (a.n_spans - 1)));
  switch (a.feature) {
    case kLinFeatOrthant: return launch_span_feat<kLinFeatOrthant>(a, grid, stream);
    case kLinFeatLorentz: return launch_span_feat<kLinFeatLorentz>(a, grid, stream);
    case kLinFeatIdentity: return launch_span_feat<kLinFeatIdentity>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear_readout(const LinArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.BH * a.n_spans));
  switch (a.feature) {
    case kLinFeatOrthant: return launch_readout_feat<kLinFeatOrthant>(a, grid, stream);
    case kLinFeatLorentz: return launch_readout_feat<kLinFeatLorentz>(a, grid, stream);
    case kLinFeatIdentity: return launch_readout_feat<kLinFeatIdentity>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kata
