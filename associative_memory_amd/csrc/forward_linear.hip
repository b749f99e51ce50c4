// The chunked read with linear cone features (KATA-Orthant, KATA-Lorentz) on
// the matrix cores; see the kernel comment below.
#include "mfma_common.h"

namespace kata {
namespace {

// ------------------------------------------------------------ linear cone features
//
// The chunked read with a linear feature psi (D = d = 64), the KATA-Orthant
// and KATA-Lorentz maps of the page (App. F.4), through the same three stages
// as the PSD map (Sec. 4.1 Eqs. 17-20 with the unsquared score
// psi(q) . psi(k)).  Per chunk of 64 tokens the raw K and Q rows pass through
// registers, where psi is applied in fp32 (orthant: ReLU(x) + shift per
// coordinate; Lorentz: (y, |y| (1 + s^2)), |y| summed over the 4 lanes that
// hold a row), and land in LDS as bf16 rows in the V layout (16-byte pieces
// swizzled by (row >> 1) & 7); V arrives by DMA into two buffers.  The fp32
// state [S | z] (64 features x 65) is one feature tile per wave, 5 value
// tiles of accumulators; psi(K)^T and [V | 1] operands of its update both come
// from transposing LDS reads.  Wave W reads out query tile W:
// O^T = [S|z]^T psi(Q)^T + [V|1]^T P^T, P = (psi(K) psi(Q)^T)^T masked.
constexpr int LCH = 64;       // chunk (tokens)
constexpr int LSB = DV + 8;   // bf16 row stride of the state copy [value row][feature]

struct alignas(16) LinRows {
  alignas(16) uint16_t r[LCH * 64];  // [token][64], 16-byte pieces swizzled by vswz
};

// One quarter row (16 dimensions) of K and of Q per thread: row tid / 4,
// dimensions 16 (tid % 4) .. +15.  Rows past the sequence read as zero and
// are written as zero features.
template <int FEAT, bool WITH_Q>
struct LinStage {
  u32x4 k[2];
  u32x4 q[2];

  __device__ __forceinline__ void load(const ChunkSrc& src, int tid) {
    const int off = (tid >> 2) * 128 + 32 * (tid & 3);
    k[0] = __builtin_amdgcn_raw_buffer_load_b128(src.k, off, 0, 0);
    k[1] = __builtin_amdgcn_raw_buffer_load_b128(src.k, off + 16, 0, 0);
    if constexpr (WITH_Q) {
      q[0] = __builtin_amdgcn_raw_buffer_load_b128(src.q, off, 0, 0);
      q[1] = __builtin_amdgcn_raw_buffer_load_b128(src.q, off + 16, 0, 0);
    }
  }

  // psi of one quarter row, written to its swizzled place
  static __device__ __forceinline__ void put(uint16_t* rows, const u32x4 (&x)[2], int tid, bool valid,
                                             float shift) {
    const int row = tid >> 2, qq = tid & 3;
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

  __device__ __forceinline__ void store(LinRows& kr, LinRows* qr, int tid, int64_t valid_rows,
                                        float shift) const {
    const bool valid = (tid >> 2) < valid_rows;
    put(kr.r, k, tid, valid, shift);
    if constexpr (WITH_Q) put(qr->r, q, tid, valid, shift);
  }
};

// 16-byte row operand: row t, dimensions 32 kf + 8 g .. +7
__device__ __forceinline__ u32x4 lin_row_op(const uint16_t* rows, int t, int kf, int g) {
  return *reinterpret_cast<const u32x4*>(&rows[t * 64 + 8 * ((4 * kf + g) ^ vswz(t))]);
}

// wave W's share of a chunk's V transfer (8 pieces of 8 rows, 2 per wave)
template <int W>
__device__ __forceinline__ void dma_lin_v(LinRows& b, const ChunkSrc& src, int lane) {
#pragma unroll
  for (int j = W; j < LCH / 8; j += 4) {
    const int t = 8 * j + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.r[8 * j * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
}

// acc[i] += psi(K)^T [V | 1] for feature tile W over the chunk
template <int W>
__device__ __forceinline__ void lin_state_update(f32x4 (&acc)[NDT], const LinRows& kr, const LinRows& vb,
                                                 const TrOffsets& to, const u32x4& bones) {
#pragma unroll
  for (int s = 0; s < LCH / 32; ++s) {
    const u32x4 ak = tr_operand<64>(kr.r, to.v[W], s);
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const u32x4 bv = i < NDT - 1 ? tr_operand<DV>(vb.r, to.v[i], s) : bones;
      acc[i] = mfma(ak, bv, acc[i]);
    }
  }
}

// workspace layout of a span state: [feature tile][value tile][lane] f32x4
__device__ __forceinline__ int lin_state_off(int W, int i, int lane) { return ((W * NDT + i) * 64 + lane) * 4; }

template <int FEAT>
__device__ __forceinline__ void lin_span_body(const LinArgs& a) {
  __shared__ LinRows kr;
  __shared__ LinRows v0;
  __shared__ LinRows v1;
  __shared__ alignas(16) uint16_t ones[128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nsp = a.n_spans - 1;  // the last span's sum is not needed
  const int64_t bh = blockIdx.x / nsp;
  const int64_t sp = blockIdx.x - bh * nsp;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * LCH;
  const int64_t end = (a.T < first + a.G * LCH) ? a.T : first + a.G * LCH;
  if (tid < 128) ones[tid] = tid < 64 ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);

  with_wave<4>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const int g = lane >> 4, r = lane & 15;
    const TrOffsets to = tr_offsets(lane);
    f32x4 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto src = [&](int64_t c0) { return chunk_src<64, LCH>(nullptr, a.k, a.v, tok0, c0, end); };
    LinStage<FEAT, false> st;
    st.load(src(first), tid);
    dma_lin_v<W>(v0, src(first), lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    st.store(kr, nullptr, tid, end - first, a.shift);
    __syncthreads();
    const u32x4 bones = *reinterpret_cast<const u32x4*>(&ones[(r > 0 ? 64 : 0) + 8 * g]);
    // chunk loop, unrolled over the two V buffers
    for (int64_t c0 = first; c0 < end; c0 += 2 * LCH) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * LCH;
        if (c >= end) break;
        LinRows& cur = u == 0 ? v0 : v1;
        LinRows& nxt = u == 0 ? v1 : v0;
        const bool more = c + LCH < end;
        if (more) {
          st.load(src(c + LCH), tid);
          dma_lin_v<W>(nxt, src(c + LCH), lane);
        }
        lin_state_update<W>(acc, kr, cur, to, bones);
        barrier_lds();
        if (more) {
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          st.store(kr, nullptr, tid, end - (c + LCH), a.shift);
        }
        barrier_lds();
      }
    }
    float* dst = a.ws + (bh * a.n_spans + sp) * kLinStateFloats;
#pragma unroll
    for (int i = 0; i < NDT; ++i) *reinterpret_cast<f32x4*>(&dst[lin_state_off(W, i, lane)]) = acc[i];
  });
}

template <int FEAT>
__global__ __launch_bounds__(256, 2) void lin_span_kernel(LinArgs a) {
  lin_span_body<FEAT>(a);
}

// the bf16 state copy [value row][feature] for the readout: rows 0..63 are
// S^T, row 64 is z, row 65 stays zero
template <int W>
__device__ __forceinline__ void lin_write_sb(uint16_t* sb, const f32x4 (&acc)[NDT], int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < NDT - 1; ++i) {
    uint2 x;
    x.x = pack2(acc[i][0], acc[i][1]);
    x.y = pack2(acc[i][2], acc[i][3]);
    *reinterpret_cast<uint2*>(&sb[(16 * i + r) * LSB + 16 * W + 4 * g]) = x;
  }
  if (r == 0) {
    uint2 x;
    x.x = pack2(acc[NDT - 1][0], acc[NDT - 1][1]);
    x.y = pack2(acc[NDT - 1][2], acc[NDT - 1][3]);
    *reinterpret_cast<uint2*>(&sb[DV * LSB + 16 * W + 4 * g]) = x;
  }
}

template <int FEAT>
__device__ __forceinline__ void lin_readout_body(const LinArgs& a) {
  __shared__ LinRows kr;
  __shared__ LinRows qr;
  __shared__ LinRows v0;
  __shared__ LinRows v1;
  __shared__ alignas(16) uint16_t sb[(DV + 2) * LSB];
  __shared__ alignas(16) uint16_t ones[128];
  __shared__ alignas(16) uint16_t Ob[4][16 * OB_LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / a.n_spans;
  const int64_t sp = blockIdx.x - bh * a.n_spans;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * LCH;
  const int64_t end = (a.T < first + a.G * LCH) ? a.T : first + a.G * LCH;
  if (tid < 128) ones[tid] = tid < 64 ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);
  if (tid < LSB / 8) *reinterpret_cast<uint4*>(&sb[(DV + 1) * LSB + 8 * tid]) = make_uint4(0, 0, 0, 0);

  with_wave<4>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const int g = lane >> 4, r = lane & 15;
    bool keep[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) keep[j] = 4 * g + j <= r;
    const TrOffsets to = tr_offsets(lane);
    f32x4 acc[NDT];
    if (a.n_spans > 1) {
      const float* P = a.ws + (bh * a.n_spans + sp) * kLinStateFloats;
#pragma unroll
      for (int i = 0; i < NDT; ++i) acc[i] = *reinterpret_cast<const f32x4*>(&P[lin_state_off(W, i, lane)]);
    } else {
#pragma unroll
      for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto src = [&](int64_t c0) { return chunk_src<64, LCH>(a.q, a.k, a.v, tok0, c0, end); };
    LinStage<FEAT, true> st;
    st.load(src(first), tid);
    dma_lin_v<W>(v0, src(first), lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    lin_write_sb<W>(sb, acc, lane);
    st.store(kr, &qr, tid, end - first, a.shift);
    __syncthreads();
    const u32x4 bones = *reinterpret_cast<const u32x4*>(&ones[(r > 0 ? 64 : 0) + 8 * g]);
    uint16_t* ob = Ob[W];
    for (int64_t c0 = first; c0 < end; c0 += 2 * LCH) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * LCH;
        if (c >= end) break;
        LinRows& cur = u == 0 ? v0 : v1;
        LinRows& nxt = u == 0 ? v1 : v0;
        const bool more = c + LCH < end;
        // the query tile's operands, then the next chunk's loads
        u32x4 qop[2];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) qop[kf] = lin_row_op(qr.r, 16 * W + r, kf, g);
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          st.load(src(c + LCH), tid);
          dma_lin_v<W>(nxt, src(c + LCH), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        // inter-chunk term: [S|z]^T psi(Q)^T
        f32x4 o[NDT];
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kf = 0; kf < 2; ++kf) {
            const u32x4 as = *reinterpret_cast<const u32x4*>(&sb[vrow(i, r) * LSB + 32 * kf + 8 * g]);
            o[i] = mfma(as, qop[kf], o[i]);
          }
        }
        // intra-chunk term over the key steps up to the diagonal, and the
        // state update over the whole chunk
#pragma unroll
        for (int s = 0; s < LCH / 32; ++s) {
          u32x4 bv[NDT];
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) bv[i] = tr_operand<DV>(cur.r, to.v[i], s);
          bv[NDT - 1] = bones;
          if (2 * s <= W) {
            float p[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int kt = 2 * s + h;
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = 0.f;
              if (kt > W) continue;
              f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kf = 0; kf < 2; ++kf) sc = mfma(lin_row_op(kr.r, 16 * kt + r, kf, g), qop[kf], sc);
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = (kt < W || keep[j]) ? sc[j] : 0.f;
            }
            const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                              pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
            for (int i = 0; i < NDT; ++i) o[i] = mfma(bv[i], pf, o[i]);
          }
          const u32x4 ak = tr_operand<64>(kr.r, to.v[W], s);
#pragma unroll
          for (int i = 0; i < NDT; ++i) acc[i] = mfma(ak, bv[i], acc[i]);
        }
        // normalise, stage the 16 x 64 tile, store it as 1 KB of rows
        {
          const __amdgpu_buffer_rsrc_t dst = rows_rsrc(a.out, tok0 + c, end - c < LCH ? end - c : LCH, 2 * DV);
          const float den = __shfl(o[NDT - 1][0], r);
          const float inv = __builtin_amdgcn_rcpf(den + a.eps);
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) {
            uint2 x;
            x.x = pack2(o[i][0] * inv, o[i][1] * inv);
            x.y = pack2(o[i][2] * inv, o[i][3] * inv);
            *reinterpret_cast<uint2*>(&ob[r * OB_LD + 16 * i + 4 * g]) = x;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + (lane >> 3);
            const uint4 x = *reinterpret_cast<const uint4*>(&ob[row * OB_LD + 8 * (lane & 7)]);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, dst,
                                                   (16 * W + row) * (2 * DV) + 16 * (lane & 7), 0, 0);
          }
        }
        barrier_lds();
        if (more) {
          lin_write_sb<W>(sb, acc, lane);
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          st.store(kr, &qr, tid, end - (c + LCH), a.shift);
        }
        barrier_lds();
      }
    }
  });
}

template <int FEAT>
__global__ __launch_bounds__(256, 2) void lin_readout_kernel(LinArgs a) {
  lin_readout_body<FEAT>(a);
}

}  // namespace

hipError_t launch_linear_span_state(const LinArgs& a, hipStream_t stream) {
  if (a.n_spans < 2) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.BH * (a.n_spans - 1)));
  if (a.feature == kLinFeatOrthant) {
    lin_span_kernel<kLinFeatOrthant><<<grid, 256, 0, stream>>>(a);
  } else if (a.feature == kLinFeatLorentz) {
    lin_span_kernel<kLinFeatLorentz><<<grid, 256, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_linear_readout(const LinArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.BH * a.n_spans));
  if (a.feature == kLinFeatOrthant) {
    lin_readout_kernel<kLinFeatOrthant><<<grid, 256, 0, stream>>>(a);
  } else if (a.feature == kLinFeatLorentz) {
    lin_readout_kernel<kLinFeatLorentz><<<grid, 256, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kata
