// The quadratic (O(T^2)) form of the causal read on the matrix cores; see the
// kernel comment below.
#include "mfma_common.h"

namespace kata {
namespace {

// ------------------------------------------------------------ quadratic forward
//
// The O(T^2) form of the read, Eq. 2 of the KATA page evaluated directly (its
// flash-style "quadratic" operating point, Sec. 4): per block of 128 queries,
// the key blocks up to the diagonal stream through LDS (DMA, two buffers);
// each gives the squared scores on the matrix cores, masked only on the
// diagonal block, and adds P [V | 1] to fp32 accumulators that stay in
// registers.  No state, no workspace.  Wave W owns query tiles W and 7 - W.
//
// Scores follow the KATA-Mg block family of Sec. 4.1: the d dimensions split
// into g = DK / M blocks of width M and the score is sum_a (q_a . k_a)^2
// (g = 1: the full map's (q . k)^2).  A score operand is a set of pieces:
// at M = 16 one 16x16x16 product per block (4 dimensions per lane), otherwise
// 16x16x32 products over 32-dimension pieces, chained within a block.
constexpr int QB = 128;

template <int DK, int M>
struct QkOp {
  static constexpr bool K16 = (M == 16);
  static constexpr int NP = K16 ? DK / 16 : DK / 32;  // pieces per operand
  static constexpr int PPB = K16 ? 1 : M / 32;         // pieces per block
  using Piece = typename ScoreOpT<K16 ? 16 : 32>::type;
  Piece p[NP];
  // first dimension of piece i held by lane group g
  static constexpr __device__ int col(int i, int g) { return K16 ? 16 * i + 4 * g : 32 * i + 8 * g; }
};

// sum over blocks of the squared score tile [key 4g + j][query r]
template <int DK, int M>
__device__ __forceinline__ void block_sq_scores(const QkOp<DK, M>& k, const QkOp<DK, M>& q, float (&p)[4]) {
  using Op = QkOp<DK, M>;
#pragma unroll
  for (int b = 0; b < Op::NP / Op::PPB; ++b) {
    f32x4 sc;
    if constexpr (Op::K16) {
      sc = score_mfma<16>(k.p[b], q.p[b]);
    } else {
      sc = mfma(k.p[b * Op::PPB], q.p[b * Op::PPB], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int j = 1; j < Op::PPB; ++j) sc = mfma(k.p[b * Op::PPB + j], q.p[b * Op::PPB + j], sc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = b == 0 ? sc[j] * sc[j] : __builtin_fmaf(sc[j], sc[j], p[j]);
  }
}

// K rows in LDS hold their 16-byte pieces XOR-swizzled by the row, so that
// the 16 rows one operand read touches fall in distinct banks:
// piece c of row r sits at c ^ ksw(r).
template <int DK>
__device__ __forceinline__ int ksw(int r) {
  constexpr int SH = DK == 16 ? 3 : (DK == 32 ? 2 : 1);  // log2(128 / DK)
  return (r >> SH) & (DK / 8 - 1);
}

template <int DK>
struct alignas(16) QuadTile {
  alignas(16) uint16_t v[QB * DV];  // [key][value column], swizzled
  alignas(16) uint16_t k[QB * DK];  // [key][dimension], swizzled
};

template <int DK, int W>
__device__ __forceinline__ void dma_quad(QuadTile<DK>& b, const ChunkSrc& src, int lane) {
#pragma unroll
  for (int j = W; j < QB / 8; j += 4) {
    const int t = 8 * j + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.v[8 * j * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
  constexpr int PPR = 2 * DK / 16;  // 16-byte pieces per K row
  constexpr int RPI = 64 / PPR;     // K rows per 1 KB transfer
#pragma unroll
  for (int j = W; j < QB / RPI; j += 4) {
    const int t = RPI * j + lane / PPR;
    const int c = (lane % PPR) ^ ksw<DK>(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, KATA_LDS(&b.k[RPI * j * DK]), 16, t * (2 * DK) + 16 * c,
                                             0, 0, 0);
  }
}

template <int DK, int M>
__device__ __forceinline__ QkOp<DK, M> quad_key_op(const QuadTile<DK>& b, int row, int g) {
  using Op = QkOp<DK, M>;
  Op op;
#pragma unroll
  for (int i = 0; i < Op::NP; ++i) {
    const int col = Op::col(i, g);
    const uint16_t* at = &b.k[row * DK + 8 * ((col >> 3) ^ ksw<DK>(row)) + (col & 7)];
    op.p[i] = *reinterpret_cast<const typename Op::Piece*>(at);
  }
  return op;
}

// one key block against the wave's two query tiles; DIAG: the block holding
// the queries themselves (causal mask, fully masked tiles skipped)
// `after_k` runs once the block's key operands are in registers (the next
// block's transfer is issued there: any earlier, the compiler's wait counts
// make these reads wait for it)
template <int DK, int M, int W, bool DIAG, class H>
__device__ __forceinline__ void quad_block(f32x4 (&o)[2][NDT], const QuadTile<DK>& b,
                                           const QkOp<DK, M> (&qf)[2], const bool (&keep)[4],
                                           const TrOffsets& to, const u32x4& bones, int lane,
                                           const H& after_k) {
  constexpr int qt[2] = {W, 7 - W};
  constexpr int qt_max = qt[0] > qt[1] ? qt[0] : qt[1];
  constexpr int NS = DIAG ? qt_max / 2 + 1 : QB / 32;  // 32-key steps read
  const int g = lane >> 4, r = lane & 15;
  QkOp<DK, M> kall[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) kall[s][h] = quad_key_op<DK, M>(b, 16 * (2 * s + h) + r, g);
  }
  after_k();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 bv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) bv[dt] = tr_operand<DV>(b.v, to.v[dt], s);
    bv[NDT - 1] = bones;
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
      if (DIAG && 2 * s > qt[slot]) continue;
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * s + h;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[h][j] = 0.f;
        if (DIAG && kt > qt[slot]) continue;
        block_sq_scores<DK, M>(kall[s][h], qf[slot], p[h]);
        if (DIAG && kt == qt[slot]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) p[h][j] = keep[j] ? p[h][j] : 0.f;
        }
      }
      const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                        pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[slot][i] = mfma(bv[i], pf, o[slot][i]);
    }
  }
}

// query blocks per group of heads in the grid order (two per CU)
constexpr int64_t kQuadGroupWorkgroups = 512;

template <int DK, int M>
__device__ __forceinline__ void quad_body(const QuadArgs& a) {
  using Op = QkOp<DK, M>;
  __shared__ QuadTile<DK> x0;
  __shared__ QuadTile<DK> x1;
  __shared__ alignas(16) uint16_t ones[128];
  __shared__ alignas(16) uint16_t Ob[4][16 * OB_LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nqb = (a.T + QB - 1) / QB;
  // Heads go in groups of about kQuadGroupWorkgroups query blocks (one
  // round of two workgroups per CU), so the resident workgroups share the
  // K and V of few heads.  Within a group the query blocks are ranked by
  // length (rank r: block nqb - 1 - r / hg of the group's head r mod hg);
  // the first half of the group takes ranks ascending, the second half
  // descending from the shortest, so the two workgroups a CU receives (j and
  // j + half) carry about the same number of key blocks together.
  const int64_t hpg = nqb >= kQuadGroupWorkgroups ? 1 : kQuadGroupWorkgroups / nqb;
  const int64_t idx = blockIdx.x;
  const int64_t grp = idx / (hpg * nqb), j = idx - grp * hpg * nqb;
  const int64_t hg = a.BH - grp * hpg < hpg ? a.BH - grp * hpg : hpg;  // heads in this group
  const int64_t nwg = hg * nqb, half = (nwg + 1) / 2;
  const int64_t rank = j < half ? j : nwg - 1 - (j - half);
  const int64_t bh = grp * hpg + rank % hg;
  const int64_t qb = nqb - 1 - rank / hg;
  const int64_t tok0 = bh * a.T;
  const int64_t q0 = qb * QB;
  const int64_t kend = (a.T < q0 + QB) ? a.T : q0 + QB;  // keys [0, kend) are read
  if (tid < 128) ones[tid] = tid < 64 ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);

  with_wave<4>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int qt[2] = {W, 7 - W};
    const int g = lane >> 4, r = lane & 15;
    bool keep[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) keep[j] = 4 * g + j <= r;
    const TrOffsets to = tr_offsets(lane);
    // the wave's query score operands, straight from HBM (rows past T read 0)
    const __amdgpu_buffer_rsrc_t qsrc = rows_rsrc(a.q, tok0 + q0, a.T - q0 < QB ? a.T - q0 : QB, 2 * DK);
    Op qf[2];
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
#pragma unroll
      for (int i = 0; i < Op::NP; ++i) {
        const int off = (16 * qt[slot] + r) * (2 * DK) + 2 * Op::col(i, g);
        if constexpr (Op::K16) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b64(qsrc, off, 0, 0);
          qf[slot].p[i] = uint2{x[0], x[1]};
        } else {
          qf[slot].p[i] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, off, 0, 0);
        }
      }
    }
    f32x4 o[2][NDT];
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[slot][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto src = [&](int64_t kb) { return chunk_src<DK, QB>(nullptr, a.k, a.v, tok0, kb * QB, kend); };
    dma_quad<DK, W>(x0, src(0), lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const u32x4 bones = *reinterpret_cast<const u32x4*>(&ones[(r > 0 ? 64 : 0) + 8 * g]);
    auto prefetch = [&](QuadTile<DK>& nxt, int64_t kb) {
      return [&src, lane, kb, p = &nxt]() {
        __builtin_amdgcn_sched_barrier(0);
        dma_quad<DK, W>(*p, src(kb), lane);
        __builtin_amdgcn_sched_barrier(0);
      };
    };
    for (int64_t kb = 0; kb < qb; kb += 2) {
      quad_block<DK, M, W, false>(o, x0, qf, keep, to, bones, lane, prefetch(x1, kb + 1));
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      barrier_lds();
      if (kb + 1 < qb) {
        quad_block<DK, M, W, false>(o, x1, qf, keep, to, bones, lane, prefetch(x0, kb + 2));
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        barrier_lds();
      }
    }
    // the diagonal block: in x0 when qb is even, in x1 when odd
    if (qb & 1) {
      quad_block<DK, M, W, true>(o, x1, qf, keep, to, bones, lane, NoHook{});
    } else {
      quad_block<DK, M, W, true>(o, x0, qf, keep, to, bones, lane, NoHook{});
    }
    // normalise; stage each 16 x 64 tile and store it as 1 KB contiguous rows
    const __amdgpu_buffer_rsrc_t dst = rows_rsrc(a.out, tok0 + q0, a.T - q0 < QB ? a.T - q0 : QB, 2 * DV);
    uint16_t* ob = Ob[W];
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
      const float den = __shfl(o[slot][NDT - 1][0], r);
      const float inv = __builtin_amdgcn_rcpf(den + a.eps);
#pragma unroll
      for (int i = 0; i < NDT - 1; ++i) {
        uint2 x;
        x.x = pack2(o[slot][i][0] * inv, o[slot][i][1] * inv);
        x.y = pack2(o[slot][i][2] * inv, o[slot][i][3] * inv);
        *reinterpret_cast<uint2*>(&ob[r * OB_LD + 16 * i + 4 * g]) = x;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + (lane >> 3);
        const uint4 x = *reinterpret_cast<const uint4*>(&ob[row * OB_LD + 8 * (lane & 7)]);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, dst,
                                               (16 * qt[slot] + row) * (2 * DV) + 16 * (lane & 7), 0, 0);
      }
    }
  });
}

template <int DK, int M>
__global__ __launch_bounds__(256, 2) void quad_kernel(QuadArgs a) {
  quad_body<DK, M>(a);
}

}  // namespace

hipError_t launch_forward_quadratic_mfma(const QuadArgs& a, hipStream_t stream) {
  const int64_t nqb = (a.T + QB - 1) / QB;
  dim3 grid(static_cast<unsigned>(a.BH * nqb));
  const int m = a.g > 0 ? a.d / a.g : 0;
  if (a.d == 16 && m == 16) {
    quad_kernel<16, 16><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 32 && m == 32) {
    quad_kernel<32, 32><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 32 && m == 16) {
    quad_kernel<32, 16><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 64 && m == 64) {
    quad_kernel<64, 64><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 64 && m == 32) {
    quad_kernel<64, 32><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 64 && m == 16) {
    quad_kernel<64, 16><<<grid, 256, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kata
