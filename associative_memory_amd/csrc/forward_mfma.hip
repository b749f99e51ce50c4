// Matrix-core (bf16 MFMA, fp32 accumulate) kernels of the chunked forward for
// dv = 64 and head dim d = 16 (D = 136) or d = 32 (D = 528) -- the KATA page,
// Sec. 4.1 Eqs. 17-20: per chunk c of a span,
//   O_c = [phi_q(Q_c) S + ((Q_c K_c^T)^2 * M) V_c] / [phi_q(Q_c) z + ((Q_c K_c^T)^2 * M) 1 + eps]
//   S  += phi_k(K_c)^T V_c,   z += phi_k(K_c)^T 1
// with the incoming (S, z) of the span taken from the exclusive prefix over
// span sums (App. E.1 three-stage pipeline).
//
// Layout decisions (all private to the forward):
//  * Features.  The D products x_a x_b (a <= b) are placed on feature
//    positions p = 32*ks + 8*g + i (ks: 32-wide MFMA k-step, g: lane group of
//    the 16x16x32 operand layout, i: slot).  Group g holds the pairs of group
//    0 shifted by g*d/4 (mod d) in both indices: every orbit of that shift
//    has 4 pairs, except the d/4 orbits {(x, x+d/2), (x+d/4, x+3d/4)} of 2.
//    A lane then builds its query-feature operand from its own query row read
//    rotated by g*d/4, with compile-time pair indices: phi(Q) never goes
//    through LDS.  Key features are built from sqrt(2) k (fp32), so every
//    key feature carries weight 2; query features carry 1 off the diagonal
//    and 1/2 on it, so phi_q . phi_k = (q.k)^2 and only the few diagonal
//    query features pay an extra multiply.
//  * Denominators.  In the register-staged kernels (d = 32, the block maps)
//    they ride through the MFMAs: V gets a column of ones (value tile 4), so
//    P.1 and phi_q.z come out of the same products as the numerators.  At
//    d = 16 (DMA kernels) a ones column would cost 9 products per 32 keys for
//    16 useful values; there z is carried as the key Gram matrix
//    Z = sum_s k_s k_s^T (one product per 32 keys), phi_q.z = q^T Z q, and
//    P.1 is summed on the vector ALU.  Either way the span state stores z as
//    a feature vector after the value tiles.
//  * Tokens inside each 32-token k-step are stored in the order in which a
//    pair of 16x16 score accumulators hands keys to the next product (the two
//    16-key halves interleaved in groups of 4), so squared scores feed P.V
//    straight from registers.
//  * The fp32 state (feature tiles x 5 value tiles) lives in registers, split
//    across the waves by feature tile; a bf16 copy in LDS is the operand of
//    the readout, which is split across waves by query tile (and, for d = 32,
//    by value tiles) and computed transposed, O^T = [S|z]^T phi_q^T + [V|1]^T P^T,
//    so a lane holds 4 consecutive value columns of one query.
#include <type_traits>

#include "kernels.h"
#include "mfma_common.h"

namespace kata {
namespace {

// ------------------------------------------------------------ feature schedule

// Feature maps of the chunked read are keyed by an id FM (the schedule,
// configuration and kernels below take it where a head width would be):
//   16, 32   the full rank-one map at d = 16, 32;
//   64       KATA-M4 at d = 64 (Sec. 4.1): four blocks of 16 dimensions, the
//            136 pairs of one block per lane group (group g holds block g,
//            the rotation by SH = 16 below), 544 feature positions; only pairs
//            inside a block carry features, the score is sum_a (q_a . k_a)^2;
//   100 + s  slice s (0..3) of the full map at d = 64 (KATA-M1): the orbits of
//            its 2,080 pairs under the rotation, 136 per slice;
//   200 + s  slice s (0..1) of KATA-M2 at d = 64 (two blocks of 32).  Q and K
//            are staged with dimension quarters 1 and 2 swapped, so the blocks
//            sit on staged quarters {0, 2} and {1, 3} and the rotation by 16
//            per lane group maps each block onto the other.
// A sliced map keeps each slice's state in its own workgroups; the slices run
// one after another and add their partial reads (fp32) before normalising.
constexpr int fm_dk(int fm) { return fm < 64 ? fm : 64; }
constexpr int fm_family(int fm) { return fm < 100 ? fm : (fm / 100) * 100; }
constexpr int fm_slice(int fm) { return fm < 100 ? 0 : fm % 100; }
constexpr int fm_slices(int fm) { return fm_family(fm) == 100 ? 4 : (fm_family(fm) == 200 ? 2 : 1); }

template <int DK>
constexpr bool kBlockMap = DK == 64;

// staged position of dimension x (KATA-M2 swaps quarters 1 and 2)
template <int FM>
constexpr int staged_dim(int x) {
  if constexpr (fm_family(FM) == 200) {
    const int q = x >> 4;
    return ((q == 1 ? 2 : (q == 2 ? 1 : q)) << 4) | (x & 15);
  } else {
    return x;
  }
}

// orbit representatives of the pairs (i <= j, staged frame) of the d = 64
// sliced maps under the shift by 16 per lane group, and the slices' bounds.
// KATA-M1 groups them by the quarter distance of the pair, which the shift
// keeps: slice 0 the pairs inside quarter 0 (136), slices 1 and 2 the pairs
// between quarters 0 and 1 (i < 8, i >= 8: 128 each), slice 3 the pairs
// between quarters 0 and 2 (136, the 16 pairs (x, x + 32) with orbits of
// size 2), so a lane needs at most 32 of its query's dimensions per slice.
// KATA-M2 (blocks are the staged quarters of equal parity) takes its 272 orbits
// size-4 first, in two slices of 136.
template <int FAM>
struct Orbits64 {
  int n4 = 0, n = 0;
  int start[5] = {};  // slice s holds entries [start[s], start[s + 1])
  int8_t a[1056] = {};
  int8_t b[1056] = {};
  bool pair2[1056] = {};
};

template <int FAM>
constexpr Orbits64<FAM> make_orbits64() {
  Orbits64<FAM> o;
  if constexpr (FAM == 100) {
    auto add = [&o](int i, int j, bool two) {
      o.a[o.n] = static_cast<int8_t>(i);
      o.b[o.n] = static_cast<int8_t>(j);
      o.pair2[o.n] = two;
      ++o.n;
      if (!two) ++o.n4;
    };
    for (int i = 0; i < 16; ++i)
      for (int j = i; j < 16; ++j) add(i, j, false);
    o.start[1] = o.n;
    for (int i = 0; i < 8; ++i)
      for (int j = 16; j < 32; ++j) add(i, j, false);
    o.start[2] = o.n;
    for (int i = 8; i < 16; ++i)
      for (int j = 16; j < 32; ++j) add(i, j, false);
    o.start[3] = o.n;
    for (int u = 0; u < 16; ++u)
      for (int x = 0; x <= u; ++x) add(x, u + 32, x == u);
    o.start[4] = o.n;
    return o;
  }
  bool used[64][64] = {};
  int n4 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < 64; ++i) {
      for (int j = i; j < 64; ++j) {
        if (FAM == 200 && ((i >> 4) & 1) != ((j >> 4) & 1)) continue;
        if (used[i][j]) continue;
        int size = 0;
        for (int g = 0; g < 4; ++g) {
          int x = (i + 16 * g) % 64, y = (j + 16 * g) % 64;
          if (x > y) { const int t = x; x = y; y = t; }
          bool dup = false;
          for (int h = 0; h < g; ++h) {
            int u = (i + 16 * h) % 64, w = (j + 16 * h) % 64;
            if (u > w) { const int t = u; u = w; w = t; }
            if (u == x && w == y) dup = true;
          }
          if (!dup) ++size;
        }
        if ((pass == 0) != (size == 4)) continue;
        for (int g = 0; g < 4; ++g) {
          int x = (i + 16 * g) % 64, y = (j + 16 * g) % 64;
          if (x > y) { const int t = x; x = y; y = t; }
          used[x][y] = true;
        }
        o.a[o.n] = static_cast<int8_t>(i);
        o.b[o.n] = static_cast<int8_t>(j);
        o.pair2[o.n] = size == 2;
        ++o.n;
        if (size == 4) ++n4;
      }
    }
  }
  o.n4 = n4;
  o.start[1] = 136;
  o.start[2] = o.n;
  return o;
}

template <int FAM>
constexpr Orbits64<FAM> kOrbits64 = make_orbits64<FAM>();

template <int FM>
constexpr int slice_entries() {
  if constexpr (FM >= 100) {
    constexpr auto& o = kOrbits64<fm_family(FM)>;
    return o.start[fm_slice(FM) + 1] - o.start[fm_slice(FM)];
  } else {
    return 0;
  }
}

template <int DK>
struct Schedule {
  static constexpr int SH = fm_dk(DK) / 4;  // index shift per lane group
  // orbit representatives (block map: the pairs of one block; slices: the
  // slice's share of the orbit list)
  static constexpr int NE = DK >= 100 ? slice_entries<DK>()
                            : kBlockMap<DK> ? 16 * 17 / 2 : (DK * (DK + 1) / 2 - DK / 2) / 4 + DK / 4;
  static constexpr int NKS = (NE + 7) / 8;                              // 32-wide feature k-steps
  static constexpr int NPOS = 32 * NKS;                                 // feature positions
  int8_t a[8 * NKS];
  int8_t b[8 * NKS];
  bool pair2[8 * NKS];  // orbit of size 2: only lane groups 0 and 1 carry it
};

template <int DK>
constexpr Schedule<DK> make_schedule() {
  Schedule<DK> s{};
  constexpr int SH = Schedule<DK>::SH;
  if constexpr (DK >= 100) {
    constexpr auto& o = kOrbits64<fm_family(DK)>;
    constexpr int first = o.start[fm_slice(DK)];
    for (int e = 0; e < Schedule<DK>::NE; ++e) {
      s.a[e] = o.a[first + e];
      s.b[e] = o.b[first + e];
      s.pair2[e] = o.pair2[first + e];
    }
  } else if constexpr (kBlockMap<DK>) {
    int e = 0;
    for (int i = 0; i < 16; ++i) {
      for (int j = i; j < 16; ++j, ++e) {
        s.a[e] = static_cast<int8_t>(i);
        s.b[e] = static_cast<int8_t>(j);
        s.pair2[e] = false;
      }
    }
  } else if constexpr (DK == 16) {
    // entry 4 j + x is the pair (x, x + j): lane group g then holds the pairs
    // (4 g + x, 4 g + x + j), the rows 4 g + x of the key-feature tile j
    // built by lane rotation (state update, d = 16), so a run of 4 entries
    // is one 8-byte store of the state copy.  j = 8 is the size-2 orbit.
    for (int j = 0; j <= 8; ++j) {
      for (int x = 0; x < 4; ++x) {
        s.a[4 * j + x] = static_cast<int8_t>(x);
        s.b[4 * j + x] = static_cast<int8_t>(x + j);
        s.pair2[4 * j + x] = (j == 8);
      }
    }
  } else if constexpr (DK == 32) {
    // entry 8 j + x is the pair (x, x + j), j = 0 .. 16: k-step j then holds
    // on feature tile 2 j row R the pair (R, R + j) and on tile 2 j + 1 row R
    // the pair (16 + R, 16 + R + j mod 32), which the state update builds by
    // lane rotation (lane R holds dimensions R and 16 + R of its tokens and
    // takes the partner from lane R + j of its row).  j = 16 is the size-2
    // orbit (tile 33 stays empty).
    for (int j = 0; j <= 16; ++j) {
      for (int x = 0; x < 8; ++x) {
        s.a[8 * j + x] = static_cast<int8_t>(x);
        s.b[8 * j + x] = static_cast<int8_t>(x + j);
        s.pair2[8 * j + x] = (j == 16);
      }
    }
  } else {
    bool used[DK][DK] = {};
    int n4 = 0, n2 = (DK * (DK + 1) / 2 - DK / 2) / 4;
    for (int i = 0; i < DK; ++i) {
      for (int j = i; j < DK; ++j) {
        if (used[i][j]) continue;
        int size = 0;
        for (int g = 0; g < 4; ++g) {
          int x = (i + SH * g) % DK, y = (j + SH * g) % DK;
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
  }
  for (int e = Schedule<DK>::NE; e < 8 * Schedule<DK>::NKS; ++e) {
    s.a[e] = -1; s.b[e] = -1; s.pair2[e] = false;
  }
  return s;
}

template <int DK>
constexpr Schedule<DK> kSched = make_schedule<DK>();

__constant__ Schedule<16> kSchedDev16 = make_schedule<16>();
__constant__ Schedule<32> kSchedDev32 = make_schedule<32>();
__constant__ Schedule<64> kSchedDev64 = make_schedule<64>();
__constant__ Schedule<100> kSchedDev100 = make_schedule<100>();
__constant__ Schedule<101> kSchedDev101 = make_schedule<101>();
__constant__ Schedule<102> kSchedDev102 = make_schedule<102>();
__constant__ Schedule<103> kSchedDev103 = make_schedule<103>();
__constant__ Schedule<200> kSchedDev200 = make_schedule<200>();
__constant__ Schedule<201> kSchedDev201 = make_schedule<201>();

template <int DK>
constexpr bool schedule_ok() {
  // every pair (a <= b) covered exactly once by the orbits
  bool seen[DK][DK] = {};
  int n = 0;
  for (int e = 0; e < Schedule<DK>::NE; ++e) {
    const int a = kSched<DK>.a[e], b = kSched<DK>.b[e];
    if (a < 0 || b < 0) return false;
    for (int g = 0; g < (kSched<DK>.pair2[e] ? 2 : 4); ++g) {
      int x = (a + Schedule<DK>::SH * g) % DK, y = (b + Schedule<DK>::SH * g) % DK;
      if (x > y) { int t = x; x = y; y = t; }
      if (seen[x][y]) return false;
      seen[x][y] = true;
      ++n;
    }
  }
  return n == DK * (DK + 1) / 2;
}

// block map: every pair inside a block covered once, nothing across blocks
template <int DK>
constexpr bool block_schedule_ok() {
  bool seen[DK][DK] = {};
  int n = 0;
  for (int e = 0; e < Schedule<DK>::NE; ++e) {
    for (int g = 0; g < 4; ++g) {
      const int x = kSched<DK>.a[e] + Schedule<DK>::SH * g, y = kSched<DK>.b[e] + Schedule<DK>::SH * g;
      if (x > y || y >= DK || x / 16 != y / 16 || seen[x][y]) return false;
      seen[x][y] = true;
      ++n;
    }
  }
  return n == 4 * 136;
}
static_assert(schedule_ok<16>(), "d = 16 feature schedule must cover every pair once");
static_assert(schedule_ok<32>(), "d = 32 feature schedule must cover every pair once");
static_assert(block_schedule_ok<64>(), "KATA-M4 schedule must cover every in-block pair once");

// sliced maps: the slices together cover every allowed pair once
template <int FAM>
constexpr bool sliced_ok() {
  constexpr auto& o = kOrbits64<FAM>;
  bool seen[64][64] = {};
  int n = 0;
  for (int e = 0; e < o.n; ++e) {
    for (int g = 0; g < (o.pair2[e] ? 2 : 4); ++g) {
      int x = (o.a[e] + 16 * g) % 64, y = (o.b[e] + 16 * g) % 64;
      if (x > y) { const int t = x; x = y; y = t; }
      if (seen[x][y]) return false;
      if (FAM == 200 && ((x >> 4) & 1) != ((y >> 4) & 1)) return false;
      seen[x][y] = true;
      ++n;
    }
  }
  for (int sl = 0; sl < (FAM == 100 ? 4 : 2); ++sl) {
    if (o.start[sl + 1] - o.start[sl] > 136) return false;  // one 34-tile state per slice
  }
  if (FAM == 100) return n == 2080 && o.n == 528 && o.n4 == 512 && o.start[4] == 528;
  return n == 1056 && o.n == 272 && o.n4 == 256 && o.start[2] == 272;
}
static_assert(sliced_ok<100>(), "KATA-M1 slices must cover every pair once");
static_assert(sliced_ok<200>(), "KATA-M2 slices must cover every in-block pair once");

// number of 16-position feature tiles holding at least one feature
template <int DK>
constexpr int feature_tiles() {
  int last = 0;
  for (int p = 0; p < Schedule<DK>::NPOS; ++p) {
    const int ks = p / 32, g = (p % 32) / 8, i = p % 8, e = 8 * ks + i;
    if (e < Schedule<DK>::NE && !(kSched<DK>.pair2[e] && g >= 2)) last = p;
  }
  return last / 16 + 1;
}
static_assert(feature_tiles<16>() == mfma_feature_tiles(16), "feature tile count (d = 16)");
static_assert(feature_tiles<32>() == mfma_feature_tiles(32), "feature tile count (d = 32)");
static_assert(feature_tiles<64>() == mfma_feature_tiles(64), "feature tile count (KATA-M4)");

template <int DK>
__device__ __forceinline__ const Schedule<DK>& sched_dev() {
  if constexpr (DK == 16) {
    return kSchedDev16;
  } else if constexpr (DK == 32) {
    return kSchedDev32;
  } else if constexpr (DK == 64) {
    return kSchedDev64;
  } else if constexpr (DK == 100) {
    return kSchedDev100;
  } else if constexpr (DK == 101) {
    return kSchedDev101;
  } else if constexpr (DK == 102) {
    return kSchedDev102;
  } else if constexpr (DK == 103) {
    return kSchedDev103;
  } else if constexpr (DK == 200) {
    return kSchedDev200;
  } else {
    return kSchedDev201;
  }
}

// pair (a, b) on feature position p, or a = -1 for an empty position
template <int DK>
__device__ __forceinline__ void pair_at(int p, int& a, int& b) {
  const Schedule<DK>& s = sched_dev<DK>();
  const int ks = p >> 5, o = p & 31, g = o >> 3, i = o & 7;
  const int e = 8 * ks + i;
  if (e >= Schedule<DK>::NE || (s.pair2[e] && g >= 2)) { a = -1; b = -1; return; }
  a = (s.a[e] + Schedule<DK>::SH * g) % fm_dk(DK);
  b = (s.b[e] + Schedule<DK>::SH * g) % fm_dk(DK);
}

// ------------------------------------------------------------ configuration

template <int FM_, int C_, int NW_ = mfma_waves(fm_dk(FM_))>
struct Cfg {
  static constexpr int FM = FM_;           // feature map id
  static constexpr int DK = fm_dk(FM_);    // head width
  static constexpr int NSL = fm_slices(FM_), SLICE = fm_slice(FM_);
  static constexpr int C = C_;
  static constexpr int NW = NW_;           // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int NKS = Schedule<FM>::NKS;
  static constexpr int NPOS = Schedule<FM>::NPOS;
  static constexpr int NFT = FM_ < 100 ? mfma_feature_tiles(DK) : feature_tiles<FM_>();
  static constexpr int MFT = (NFT + NW - 1) / NW;   // feature tiles per wave (max)
  // bf16 row stride of the state copy; at d = 16 (160 positions) rows of
  // 352 bytes keep the 16-byte operand reads of 16 rows x 4 lane groups free
  // of bank conflicts (7.4 cycles per read per CU against 10.9 at 336 bytes)
  static constexpr int SB_LD = DK == 16 ? NPOS + 16 : NPOS + 8;
  static constexpr int QF_LD = DK + 4;              // fp32 row stride of Q
  // bf16 row strides of K and V^T: a multiple of 16 bytes that is 2 mod 4 in
  // 16-byte units, so 16-byte reads of 16 consecutive rows by 4 lane groups
  // hit no bank twice (measured 7.2-7.4 cycles per read per CU against 10.2-10.6
  // at the next strides either side)
  static constexpr int KB_LD = DK == 16 ? 48 : DK == 32 ? 48 : 80;
  static constexpr int LDT = C == 64 ? 80 : 144;
  static constexpr int LDK = C + 4;                 // fp32 row stride of K^T
  // readout split: 4 waves take 1 or 2 query tiles each with all value tiles;
  // 8 waves take one query tile each, at chunk 64 sharing it between two
  // waves that split the value tiles
  static constexpr int NSLOT = (NW == 4 && C == 128) ? 2 : 1;  // query tiles per wave
  static constexpr int NDW = (NW == 8 && C == 64) ? 3 : NDT;   // value tiles per wave
  static constexpr int ZOFF = NFT * (NDT - 1) * 256;  // z column offset in a span state
  // whole output rows leave through a per-wave LDS tile as 16-byte stores;
  // otherwise 8-byte stores from the accumulators
  static constexpr bool STAGE_OUT = NDW == NDT;
  static_assert(NT >= 2 * C, "one thread per K row and per Q row");
  static_assert((NW == 4 || NW == 8) && (C == 64 || C == 128), "tiling");
};

// query tile of a wave's slot, balanced for the causal work
template <class CF>
__device__ __forceinline__ int query_tile(int w, int slot) {
  if constexpr (CF::NW == 4) {
    if constexpr (CF::C == 128) {
      constexpr int t[4][2] = {{0, 1}, {2, 7}, {3, 6}, {4, 5}};
      return t[w][slot];
    } else {
      return w;
    }
  } else {
    return CF::C == 64 ? (w & 3) : w;
  }
}

// value tile of a wave's readout index: all five tiles, or for two waves
// sharing a query tile {0, 1, 4} and {2, 3, 4} (both carry the denominator)
template <class CF>
__device__ __forceinline__ int value_tile(int w, int idx) {
  if constexpr (CF::NDW == NDT) {
    return idx;
  } else {
    return idx == 2 ? 4 : idx + ((w >> 2) << 1);
  }
}

template <>
struct ScoreOpT<64> {  // KATA-M4: one 16x16x16 operand per block
  struct type {
    uint2 p[4];
  };
};
template <>
struct ScoreOpT<100> {  // d = 64 sliced maps: two 16x16x32 operands
  struct type {
    u32x4 p[2];
  };
};
template <int FM>
using ScoreOp = typename ScoreOpT<(FM >= 100 ? 100 : FM)>::type;

// position of the first of 4 consecutive tokens (group tg) inside a chunk:
// within each 32-token block, token groups 0..3 sit at 8a, groups 4..7 at
// 8(a-4)+4, matching the key order of a pair of 16x16 accumulators.
__device__ __forceinline__ int group_pos(int tg) {
  const int a = tg & 7;
  return (tg >> 3) * 32 + ((a < 4) ? 8 * a : 8 * (a - 4) + 4);
}

// ------------------------------------------------------------ LDS tiles
//
// Row strides are padded so the 16-byte operand reads of 16 consecutive
// lanes (consecutive rows) land on distinct bank groups; every row starts
// 16-byte aligned so the reads stay single b128 accesses.
template <class CF>
struct alignas(16) Smem {
  // [value column][token position]; row 64 all ones and row 65 all zeros
  // (the ones-column tile [1 | 0]), written once per kernel
  alignas(16) uint16_t Vt[VROWS * CF::LDT];
  alignas(16) float Kt[(CF::DK + 1) * CF::LDK];  // [d][token position] fp32; row d is zero
};

template <class CF>
struct alignas(16) Tiles : Smem<CF> {
  alignas(16) uint16_t Kb[CF::C * CF::KB_LD];  // [token][d] bf16 (score operand)
  alignas(16) float Qf[CF::C * CF::QF_LD];     // [token][d] fp32
};

template <class CF>
struct alignas(16) SmemOut : Tiles<CF> {
  alignas(16) uint16_t Sb[VROWS * CF::SB_LD];  // [value row][feature position] bf16 state
  // per-wave 16 x 64 output tile, staged so the chunk's rows leave as
  // contiguous 16-byte stores (used when a wave owns whole output rows)
  alignas(16) uint16_t Ob[CF::STAGE_OUT ? CF::NW : 1][16 * OB_LD];
};

// score operand of row `row` from the fp32 Q tile / the bf16 K tile
// first staged dimension of piece j of lane group g: the full map at d = 64
// takes 32-dimension pieces; KATA-M2 takes block j's 8 dimensions of group g
// (staged quarters j and j + 2)
template <int FM>
__device__ __forceinline__ int piece_dim(int j, int g) {
  if constexpr (fm_family(FM) == 200) {
    return 16 * (j + 2 * (g >> 1)) + 8 * (g & 1);
  } else {
    return 32 * j + 8 * g;
  }
}

template <class CF>
__device__ __forceinline__ ScoreOp<CF::FM> score_operand(const float* Qf, int row, int g) {
  if constexpr (CF::FM >= 100) {
    ScoreOp<CF::FM> op;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float* q = &Qf[row * CF::QF_LD + piece_dim<CF::FM>(j, g)];
      const float4 x0 = *reinterpret_cast<const float4*>(q);
      const float4 x1 = *reinterpret_cast<const float4*>(q + 4);
      op.p[j] = u32x4{pack2(x0.x, x0.y), pack2(x0.z, x0.w), pack2(x1.x, x1.y), pack2(x1.z, x1.w)};
    }
    return op;
  } else if constexpr (kBlockMap<CF::FM>) {
    ScoreOp<CF::FM> op;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 x = *reinterpret_cast<const float4*>(&Qf[row * CF::QF_LD + 16 * a + 4 * g]);
      op.p[a] = uint2{pack2(x.x, x.y), pack2(x.z, x.w)};
    }
    return op;
  } else if constexpr (CF::DK == 16) {
    const float4 x = *reinterpret_cast<const float4*>(&Qf[row * CF::QF_LD + 4 * g]);
    return uint2{pack2(x.x, x.y), pack2(x.z, x.w)};
  } else {
    const float* q = &Qf[row * CF::QF_LD + 8 * g];
    const float4 x0 = *reinterpret_cast<const float4*>(q);
    const float4 x1 = *reinterpret_cast<const float4*>(q + 4);
    return u32x4{pack2(x0.x, x0.y), pack2(x0.z, x0.w), pack2(x1.x, x1.y), pack2(x1.z, x1.w)};
  }
}

template <class CF>
__device__ __forceinline__ ScoreOp<CF::FM> score_operand_bf16(const uint16_t* Kb, int row, int g) {
  if constexpr (CF::FM >= 100) {
    ScoreOp<CF::FM> op;
#pragma unroll
    for (int j = 0; j < 2; ++j) op.p[j] = *reinterpret_cast<const u32x4*>(&Kb[row * CF::KB_LD + piece_dim<CF::FM>(j, g)]);
    return op;
  } else if constexpr (kBlockMap<CF::FM>) {
    ScoreOp<CF::FM> op;
#pragma unroll
    for (int a = 0; a < 4; ++a) op.p[a] = *reinterpret_cast<const uint2*>(&Kb[row * CF::KB_LD + 16 * a + 4 * g]);
    return op;
  } else if constexpr (CF::DK == 16) {
    return *reinterpret_cast<const uint2*>(&Kb[row * CF::KB_LD + 4 * g]);
  } else {
    return *reinterpret_cast<const u32x4*>(&Kb[row * CF::KB_LD + 8 * g]);
  }
}

// ------------------------------------------------------------ chunk staging
//
// Global -> registers -> LDS for one chunk.  V: groups of 4 tokens x 8
// columns (16 B per token), written transposed; K and Q: one token row per
// thread.  Tokens at or past T read as zero (buffer range check).
// Gated read (G): a K row thread also loads its token's key factor
// 2^((beta_C - beta_t) / 2) and scales the row's fp32 copy (the state
// update's operand) by it; a Q row thread loads its token's beta_t / 2 into
// the chunk's gate row `gb`.  The bf16 K rows of the scores stay unscaled.
template <class CF, bool WITH_Q, bool G = false>
struct Stage {
  static constexpr int C = CF::C, DK = CF::DK;
  static constexpr int NVG = (C / 4) * (DV / 8);
  static constexpr int RW = DK / 8;  // 16-byte words per K/Q row
  uint4 v[4];
  uint4 kq[RW];  // one K row or, with Q, one Q row (threads [C, 2C))
  float gate;    // gated read: the key factor (K rows) or beta / 2 (Q rows)

  // K row staged by thread tid, or -1: threads [0, C) with Q; without Q the
  // last C threads, away from wave 0, which reduces the extra feature tile
  static __device__ __forceinline__ int krow(int tid) {
    if constexpr (WITH_Q) {
      return tid < C ? tid : -1;
    } else {
      return tid >= CF::NT - C ? tid - (CF::NT - C) : -1;
    }
  }

  __device__ __forceinline__ void load(const ChunkSrc& src, int tid) {
    if (tid < NVG) {
      const int tg = tid % (C / 4), cg = tid / (C / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = buf_load16(src.v, (4 * tg + r) * (2 * DV) + 16 * cg);
    }
    if constexpr (WITH_Q) {
      if (tid < 2 * C) {
        const bool is_q = tid >= C;
        const int t = is_q ? tid - C : tid;
#pragma unroll
        for (int u = 0; u < RW; ++u) kq[u] = buf_load16(is_q ? src.q : src.k, t * (2 * DK) + 16 * u);
        if constexpr (G) gate = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(is_q ? src.g : src.gk, 4 * t, 0, 0));
      }
    } else {
      const int t = krow(tid);
      if (t >= 0) {
#pragma unroll
        for (int u = 0; u < RW; ++u) kq[u] = buf_load16(src.k, t * (2 * DK) + 16 * u);
        if constexpr (G) gate = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(src.gk, 4 * t, 0, 0));
      }
    }
  }

  template <class S>
  __device__ __forceinline__ void store(S& sm, int tid, float* gb = nullptr) const {
    constexpr int LDT = CF::LDT, LDK = CF::LDK;
    if (tid < NVG) {
      const int tg = tid % (C / 4), cg = tid / (C / 4);
      const int pos = group_pos(tg);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int c = x >> 1;
        const uint32_t w0 = c == 0 ? v[0].x : c == 1 ? v[0].y : c == 2 ? v[0].z : v[0].w;
        const uint32_t w1 = c == 0 ? v[1].x : c == 1 ? v[1].y : c == 2 ? v[1].z : v[1].w;
        const uint32_t w2 = c == 0 ? v[2].x : c == 1 ? v[2].y : c == 2 ? v[2].z : v[2].w;
        const uint32_t w3 = c == 0 ? v[3].x : c == 1 ? v[3].y : c == 2 ? v[3].z : v[3].w;
        // column x of the 4 tokens: low (even x) or high (odd x) halves
        const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
        uint2 o;
        o.x = __builtin_amdgcn_perm(w1, w0, sel);
        o.y = __builtin_amdgcn_perm(w3, w2, sel);
        *reinterpret_cast<uint2*>(&sm.Vt[(8 * cg + x) * LDT + pos]) = o;
      }
    }
    uint32_t w[4 * RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      w[4 * u + 0] = kq[u].x;
      w[4 * u + 1] = kq[u].y;
      w[4 * u + 2] = kq[u].z;
      w[4 * u + 3] = kq[u].w;
    }
    if (krow(tid) >= 0) {
      // K row: fp32 transposed copy scaled by sqrt(2) (key features) and,
      // with Q, a bf16 row copy (scores)
      const int t = krow(tid);
      const int pos = group_pos(t >> 2) + (t & 3);
      const float ks = G ? kSqrt2 * gate : kSqrt2;
#pragma unroll
      for (int x = 0; x < DK; ++x) {
        sm.Kt[staged_dim<CF::FM>(x) * LDK + pos] = ks * ((x & 1) ? hi_bf16(w[x >> 1]) : lo_bf16(w[x >> 1]));
      }
      if constexpr (WITH_Q) {
#pragma unroll
        for (int u = 0; u < RW; ++u) {
          *reinterpret_cast<uint4*>(&sm.Kb[t * CF::KB_LD + staged_dim<CF::FM>(8 * u)]) = kq[u];
        }
      }
    } else if (WITH_Q && tid < 2 * C) {
      if constexpr (WITH_Q) {
        const int t = tid - C;
        if constexpr (G) gb[t] = gate;
#pragma unroll
        for (int c = 0; c < DK / 4; ++c) {
          float4 f;
          f.x = lo_bf16(w[2 * c]);
          f.y = hi_bf16(w[2 * c]);
          f.z = lo_bf16(w[2 * c + 1]);
          f.w = hi_bf16(w[2 * c + 1]);
          *reinterpret_cast<float4*>(&sm.Qf[t * CF::QF_LD + staged_dim<CF::FM>(4 * c)]) = f;
        }
      }
    }
  }
};

// constant LDS rows written once per kernel: the zero row of K^T read by empty
// feature positions, and the ones-column tile of V^T
template <class CF, class S>
__device__ __forceinline__ void init_const_rows(S& sm, int tid) {
  for (int e = tid; e < CF::LDK; e += CF::NT) sm.Kt[CF::DK * CF::LDK + e] = 0.f;
  for (int e = tid; e < 2 * CF::LDT; e += CF::NT) {
    sm.Vt[DV * CF::LDT + e] = (e < CF::LDT) ? static_cast<uint16_t>(0x3f80u) : static_cast<uint16_t>(0);
  }
}

// ------------------------------------------------------------ state update
//
// acc[m][dt] += phi_k(K_c)^T [V_c | 1 | 0] for the feature tiles ft = w + NW m
// this wave owns.  The key-feature operand (position 16 ft + r, 8 token
// slots) is built from two fp32 rows of K^T.
template <class CF>
struct KeyPairs {
  int a[CF::MFT];
  int b[CF::MFT];
};

template <class CF>
__device__ __forceinline__ KeyPairs<CF> key_pairs(int w, int r) {
  KeyPairs<CF> kp;
#pragma unroll
  for (int m = 0; m < CF::MFT; ++m) {
    const int ft = w + CF::NW * m;
    int a = -1, b = -1;
    if (ft < CF::NFT) pair_at<CF::FM>(16 * ft + r, a, b);
    // an empty position reads the zero row of K^T: its features are 0
    kp.a[m] = a < 0 ? CF::DK : a;
    kp.b[m] = b < 0 ? CF::DK : b;
  }
  return kp;
}

// lane r of each 16-lane row receives the value of lane (r + J) mod 16
template <int J>
__device__ __forceinline__ float row_rotate(float x) {
  if constexpr (J == 0) {
    return x;
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x120 + (16 - J), 0xF, 0xF, true));
  }
}

// f[i] = a[i] * (b[i] of lane (r + J) mod 16 of the row), J = 1..15, as eight
// v_mul_f32 with the row rotation in the DPP field of the first operand.
// Written with a rotating move and a multiply, about half of the d = 32
// products compiled to the two separate instructions (the compiler's folding
// of the move into its user did not take where the move was emitted far from
// the multiply); written out, the rotation costs nothing.  DPP reads a VGPR
// two wait states after a VALU write at the earliest, hence the leading s_nop
// (the inputs may have been written by the instructions just before).
template <int J>
__device__ __forceinline__ void mul_row_rotated(float (&f)[8], const float (&a)[8], const float (&b)[8]) {
  static_assert(J > 0 && J < 16, "row rotation by 1..15 lanes");
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %16, %8 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %17, %9 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %2, %18, %10 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %3, %19, %11 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %4, %20, %12 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %5, %21, %13 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %6, %22, %14 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %7, %23, %15 row_ror:%24 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]), "n"(16 - J));
}

// d = 16: key-feature tile J (J = 0..8) holds on row R the pair (R, R + J mod
// 16).  Lane (g, r) loads its own dimension r of its 8 tokens once per
// k-step and takes the partner dimension from lane r + J of its row, so the
// features of every tile come from one 32-byte read per lane and k-step.
// Rows 8..15 of tile 8 repeat rows 0..7; the state copy drops them.
// N: value tiles updated (the d = 16 DMA kernels leave out the ones-column tile)
template <int J, int N = NDT>
__device__ __forceinline__ void tile16_into(f32x4 (&dst)[NDT], const float (&kr)[8], const u32x4 (&bv)[NDT]) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = kr[i] * row_rotate<J>(kr[i]);
  const u32x4 af = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
#pragma unroll
  for (int dt = 0; dt < N; ++dt) dst[dt] = mfma(af, bv[dt], dst[dt]);
}

template <class CF, int J>
__device__ __forceinline__ void state_tile16(f32x4 (&acc)[CF::MFT][NDT], const float (&kr)[8],
                                             const u32x4 (&bv)[NDT], int w) {
  if (J % CF::NW != w) return;  // uniform per wave
  tile16_into<J>(acc[J / CF::NW], kr, bv);
}

template <class CF, int... J>
__device__ __forceinline__ void state_tiles16(f32x4 (&acc)[CF::MFT][NDT], const float (&kr)[8],
                                              const u32x4 (&bv)[NDT], int w,
                                              std::integer_sequence<int, J...>) {
  (state_tile16<CF, J>(acc, kr, bv, w), ...);
}

// (N: value tiles updated; the gated read leaves out the ones-column tile.
// HS, HO: at d >= 32 only the wave's tiles m with m % HS == HO, for span sums
// split over HS workgroups)
template <class CF, class S, int N = NDT, int HS = 1, int HO = 0>
__device__ __forceinline__ void state_update(f32x4 (&acc)[CF::MFT][NDT], const S& sm, int w, int lane,
                                             const KeyPairs<CF>& kp) {
  constexpr int LDT = CF::LDT, LDK = CF::LDK;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int ks = 0; ks < CF::C / 32; ++ks) {
    u32x4 bv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      bv[dt] = *reinterpret_cast<const u32x4*>(&sm.Vt[vrow(dt, r) * LDT + 32 * ks + 8 * g]);
    }
    if constexpr (CF::DK == 16) {
      const float* rk = &sm.Kt[r * LDK + 32 * ks + 8 * g];
      const float4 k0 = *reinterpret_cast<const float4*>(rk);
      const float4 k1 = *reinterpret_cast<const float4*>(rk + 4);
      const float kr[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      state_tiles16<CF>(acc, kr, bv, w, std::make_integer_sequence<int, CF::NFT>{});
    } else {
#pragma unroll
      for (int m = 0; m < CF::MFT; ++m) {
        if (m % HS != HO) continue;                // this workgroup's half (compile time)
        if (w + CF::NW * m >= CF::NFT) continue;  // uniform per wave
        const float* ra = &sm.Kt[kp.a[m] * LDK + 32 * ks + 8 * g];
        const float* rb = &sm.Kt[kp.b[m] * LDK + 32 * ks + 8 * g];
        const float4 a0 = *reinterpret_cast<const float4*>(ra);
        const float4 a1 = *reinterpret_cast<const float4*>(ra + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(rb);
        const float4 b1 = *reinterpret_cast<const float4*>(rb + 4);
        u32x4 af;
        af.x = pack2(a0.x * b0.x, a0.y * b0.y);
        af.y = pack2(a0.z * b0.z, a0.w * b0.w);
        af.z = pack2(a1.x * b1.x, a1.y * b1.y);
        af.w = pack2(a1.z * b1.z, a1.w * b1.w);
#pragma unroll
        for (int dt = 0; dt < N; ++dt) acc[m][dt] = mfma(af, bv[dt], acc[m][dt]);
      }
    }
  }
}

// fp32 state tiles <-> workspace.  Value tiles 0..3 in tile-native order
// ((ft*4 + dt)*64 + lane)*4 + j; the ones-column tile only carries z in its
// column 0 (lanes r == 0), stored as 16 floats per feature tile.
template <class CF>
__device__ __forceinline__ void load_state(f32x4 (&acc)[CF::MFT][NDT], const float* __restrict__ P,
                                           int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < CF::MFT; ++m) {
    const int ft = w + CF::NW * m;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (P == nullptr || ft >= CF::NFT) continue;
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) {
      const float4 x = *reinterpret_cast<const float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4);
      acc[m][dt] = f32x4{x.x, x.y, x.z, x.w};
    }
    if (r == 0) {
      const float4 x = *reinterpret_cast<const float4*>(P + CF::ZOFF + ft * 16 + 4 * g);
      acc[m][NDT - 1] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
}

// The value tiles of the wave's feature tiles summed over the n span sums at
// P0, P0 + E, ... in span order: the sums the sequential prefix forms, bit
// for bit (the z column is not read)
template <class CF>
__device__ __forceinline__ void sum_states(f32x4 (&acc)[CF::MFT][NDT], const float* __restrict__ P0,
                                           int64_t n, int w, int lane) {
#pragma unroll
  for (int m = 0; m < CF::MFT; ++m) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll 2
  for (int64_t s = 0; s < n; ++s) {
    const float* P = P0 + s * mfma_state_floats(CF::DK);
#pragma unroll
    for (int m = 0; m < CF::MFT; ++m) {
      const int ft = w + CF::NW * m;
      if (ft >= CF::NFT) continue;
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) {
        const float4 x = *reinterpret_cast<const float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4);
        acc[m][dt] += f32x4{x.x, x.y, x.z, x.w};
      }
    }
  }
}

// (WITH_Z false: the z column is written elsewhere)
// (HS, HO: only the tiles m with m % HS == HO)
template <class CF, bool WITH_Z = true, int HS = 1, int HO = 0>
__device__ __forceinline__ void store_state(const f32x4 (&acc)[CF::MFT][NDT], float* __restrict__ P,
                                            int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < CF::MFT; ++m) {
    const int ft = w + CF::NW * m;
    if (ft >= CF::NFT || m % HS != HO) continue;
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) {
      *reinterpret_cast<float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4) =
          make_float4(acc[m][dt][0], acc[m][dt][1], acc[m][dt][2], acc[m][dt][3]);
    }
    if (WITH_Z && r == 0) {
      *reinterpret_cast<float4*>(P + CF::ZOFF + ft * 16 + 4 * g) =
          make_float4(acc[m][NDT - 1][0], acc[m][NDT - 1][1], acc[m][NDT - 1][2],
                      acc[m][NDT - 1][3]);
    }
  }
}

// Column of the state copy holding rows 4g..4g+3 of feature tile ft.  At
// d = 16 tile J's row R is the pair (R, R + J), which the query schedule puts
// on k-step J/2, lane group R/4, slots 4(J%2) + R%4; otherwise tile ft covers
// columns 16 ft .. 16 ft + 15.
template <class CF>
__host__ __device__ constexpr int sb_col(int ft, int g) {
  return CF::DK == 16 ? 32 * (ft / 2) + 8 * g + 4 * (ft % 2) : 16 * ft + 4 * g;
}

// true if no feature tile writes column c of the state copy (zeroed once)
template <class CF>
__host__ __device__ constexpr bool sb_col_unused(int c) {
  if constexpr (CF::DK == 16) {
    return 2 * (c / 32) + (c % 8) / 4 >= CF::NFT;
  } else {
    return c >= 16 * CF::NFT;
  }
}
// d = 16: the unused columns are 128 + 8 i + 4 + m (i, m = 0..3), the
// positions the DMA readout zeroes directly
constexpr bool sb_unused16_ok() {
  int n = 0;
  for (int c = 0; c < Schedule<16>::NPOS; ++c) {
    const bool listed = c >= 128 && (c & 4) != 0;
    if (sb_col_unused<Cfg<16, 64>>(c) != listed) return false;
    n += listed;
  }
  return n == 16;
}
static_assert(sb_unused16_ok(), "unused state-copy columns at d = 16");

// bf16 copy of the owned state tiles into Sb[value row][feature position]
// (ND: value tiles copied; the d = 16 DMA readout keeps no z column in Sb.
// HALF_DIAG: feature tile 0, the diagonal pairs at d = 16, is stored halved,
// so the query's diagonal features need no factor 1/2.)
template <class CF, int ND = NDT, bool HALF_DIAG = false>
__device__ __forceinline__ void write_sb(uint16_t* __restrict__ Sb, const f32x4 (&acc)[CF::MFT][NDT],
                                         int w, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < CF::MFT; ++m) {
    const int ft = w + CF::NW * m;
    if (ft >= CF::NFT) continue;
    // d = 16, tile 8: rows 8..15 repeat rows 0..7 and are stored as zero
    const bool dup = CF::DK == 16 && ft == 8 && g >= 2;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      // ones-column tile: column 0 is z (row 64), the rest are zero (row 65)
      if (dt == NDT - 1 && r > 1) continue;
      uint2 o;
      const float h = HALF_DIAG && ft == 0 ? 0.5f : 1.f;
      o.x = dup ? 0u : pack2(h * acc[m][dt][0], h * acc[m][dt][1]);
      o.y = dup ? 0u : pack2(h * acc[m][dt][2], h * acc[m][dt][3]);
      *reinterpret_cast<uint2*>(&Sb[vrow(dt, r) * CF::SB_LD + sb_col<CF>(ft, g)]) = o;
    }
  }
}

// state decay of the gated read (the ones-column tile is unused there)
template <int NA, int NB>
__device__ __forceinline__ void gate_decay(f32x4 (&acc)[NA][NB], float f) {
#pragma unroll
  for (int m = 0; m < NA; ++m) {
#pragma unroll
    for (int dt = 0; dt < NB - 1; ++dt) acc[m][dt] *= f;  // the ones-column tile is unused
  }
}

// ------------------------------------------------------------ span sums

// Gated read (G): before a chunk's keys are added the state decays by the
// chunk's gate product 2^beta_C (beta_C / 2 read from the gate sums at the
// chunk's last token; every chunk of a summed span is whole), and the staged
// key rows carry their key factors.  The ones-column tile is not updated.
// NH = 2 (fewer spans than CUs): two workgroups per span, both staging the
// whole chunk; half h reduces the wave's tiles m with m % 2 == h.  Blocks b
// and b + BH (n_spans - 1) hold the two halves of a span.
template <class CF, bool G = false, int NH = 1>
__device__ __forceinline__ void span_state_mfma_body(const MfmaArgs& a) {
  constexpr int C = CF::C, DK = CF::DK;
  // two LDS tile buffers: chunk i is staged into buffer i % 2 while the
  // other buffer may still be read for chunk i - 1, so one barrier per chunk
  __shared__ Smem<CF> sm[2];
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keep it scalar so every
  // wave-dependent branch is a scalar branch, not an exec-mask region
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nsp_work = a.n_spans - 1;  // the last span's sum is never read
  const int64_t nwork = a.BH * nsp_work;
  const int hh = NH == 1 ? 0 : static_cast<int>(blockIdx.x / nwork);
  const int64_t blk = blockIdx.x - hh * nwork;
  const int64_t bh = blk / nsp_work;
  const int64_t sp = blk - bh * nsp_work;
  const int64_t tok0 = bh * a.T;

  init_const_rows<CF>(sm[0], tid);
  init_const_rows<CF>(sm[1], tid);
  auto half = [&](auto hc) {
  constexpr int H = decltype(hc)::value;
  with_wave<CF::NW>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const KeyPairs<CF> kp = key_pairs<CF>(W, lane & 15);
    f32x4 acc[CF::MFT][NDT];
    load_state<CF>(acc, nullptr, W, lane);

    const int64_t first = sp * a.G * C;
    int64_t end = first + a.G * C;
    if (end > a.T) end = a.T;
    Stage<CF, false, G> st;
    auto src = [&](int64_t c) { return chunk_src<DK, C>(nullptr, a.k, a.v, tok0, c, a.T, a.gb, a.gk); };
    st.load(src(first), tid);
    int buf = 0;
    for (int64_t c0 = first; c0 < end; c0 += C, buf ^= 1) {
      st.store(sm[buf], tid);
      if (c0 + C < end) st.load(src(c0 + C), tid);
      __syncthreads();
      if constexpr (G) {
        gate_decay(acc, __builtin_amdgcn_exp2f(2.f * a.gb[tok0 + c0 + C - 1]));
        state_update<CF, Smem<CF>, NDT - 1, NH, H>(acc, sm[buf], W, lane, kp);
      } else {
        state_update<CF, Smem<CF>, NDT, NH, H>(acc, sm[buf], W, lane, kp);
      }
    }
    store_state<CF, true, NH, H>(acc, a.ws + (bh * a.n_spans + sp) * mfma_state_floats(DK), W, lane);
  });
  };
  if (NH == 1 || hh == 0) {
    half(std::integral_constant<int, 0>{});
  } else if constexpr (NH == 2) {
    half(std::integral_constant<int, 1>{});
  }
}

template <class CF, bool G = false, int NH = 1>
__global__ __launch_bounds__(CF::NT) void span_state_mfma_kernel(MfmaArgs a) {
  span_state_mfma_body<CF, G, NH>(a);
}

// ------------------------------------------------------------ span sums, d = 16, LDS DMA
//
// The chunk goes from HBM straight into LDS (`buffer_load ... lds`, no
// registers, no VALU): raw V rows (128 B, 16-byte pieces XOR-swizzled by
// vswz(row) against bank conflicts) and raw K rows (32 B, pieces swizzled by
// ksw16(row)).  The MFMA
// operands are read back with the transposing LDS read `ds_read_b64_tr_b16`:
// in each 16-lane group, lane i receives element i % 4 of the 8 bytes
// addressed by lanes 4m + i/4 (m = 0..3), so when lane s addresses row m = s/4,
// columns 4(s % 4)..+3 of a row-major tile, lane i gets column i of 4
// consecutive rows.  The two buffers are distinct LDS variables and the loop
// is unrolled over them, so the compiler's wait counts see that a chunk
// arriving in one buffer does not alias reads of the other.
// Gated read only: half the chunk's running gate sums, beta_t / 2 (log2
// units, see gate_prep_kernel) and, in the span-sum tiles, the key factors
// 2^((beta_C - beta_t) / 2), each filled by one DMA instruction of C/4 lanes
// (entries past the sequence read as 0).  The ungated tiles carry nothing
// (empty base).  The readout tiles leave the key factors out (at C = 128
// their 2 x 512 bytes would exceed the LDS of two workgroups per CU) and
// compute them from beta.
template <int C, bool G, bool KF = G>
struct GateRows {};
template <int C>
struct GateRows<C, true, false> {
  alignas(16) float gb[C];
};
template <int C>
struct GateRows<C, true, true> {
  alignas(16) float gb[C];
  alignas(16) float gk[C];
};

template <int C, bool G = false>
struct alignas(16) DmaTile16 : GateRows<C, G> {
  static constexpr bool kKeyFactors = G;
  alignas(16) uint16_t v[C * DV];  // [token][value column], swizzled
  alignas(16) uint16_t k[C * 16];  // [token][dimension]
};

// wave W's share of the chunk's DMA: V in 1 KB pieces of 8 rows, K in 1 KB
// pieces of 32 rows; rows past the buffer resource's end arrive as zero
// the gate sums and (span sums) key factors of a chunk of C tokens: one DMA
// each, by the last two waves, lanes [0, C/4) moving 16 bytes each
template <bool G, int W, int NW, class B>
__device__ __forceinline__ void dma_gate(B& b, const ChunkSrc& src, int lane) {
  if constexpr (G && W == NW - 1) {
    constexpr int NL = static_cast<int>(sizeof(b.gb)) / 16;
    if (lane < NL) __builtin_amdgcn_raw_ptr_buffer_load_lds(src.g, KATA_LDS(&b.gb[0]), 16, 16 * lane, 0, 0, 0);
  }
  if constexpr (G && W == NW - 2 && B::kKeyFactors) {
    constexpr int NL = static_cast<int>(sizeof(b.gk)) / 16;
    if (lane < NL) __builtin_amdgcn_raw_ptr_buffer_load_lds(src.gk, KATA_LDS(&b.gk[0]), 16, 16 * lane, 0, 0, 0);
  }
}

template <int C, int W, int NW, bool G = false>
__device__ __forceinline__ void dma_chunk16(DmaTile16<C, G>& b, const ChunkSrc& src, int lane) {
#pragma unroll
  for (int j = W; j < C / 8; j += NW) {
    const int t = 8 * j + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.v[8 * j * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
#pragma unroll
  for (int j = W; j < C / 32; j += NW) {
    const int t = 32 * j + (lane >> 1);
    const int pc = (lane & 1) ^ ksw16(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, KATA_LDS(&b.k[32 * j * 16]), 16, t * 32 + 16 * pc, 0, 0, 0);
  }
  dma_gate<G, W, NW>(b, src, lane);
}

// Gated read (GatedKATA, S_t = gamma_t S_{t-1} + phi(k_t) v_t^T): over a
// chunk with running gate sums beta_t (log2 units) and total beta_C,
//   S <- 2^beta_C S + sum_s 2^(beta_C - beta_s) phi(k_s) v_s^T.
// phi is quadratic in k, so token s's key row is scaled by its key factor
// 2^((beta_C - beta_s) / 2) (computed once per token by gate_prep_kernel);
// the lane's 8 tokens are those of its transposed K operand (32 ks + 4g + m
// and 32 ks + 16 + 4g + m).

__device__ __forceinline__ void gate_keys(float (&kr)[8], const float* gk, int ks) {
  const int g = __lane_id() >> 4;
  const float4 f0 = *reinterpret_cast<const float4*>(&gk[32 * ks + 4 * g]);
  const float4 f1 = *reinterpret_cast<const float4*>(&gk[32 * ks + 16 + 4 * g]);
  const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) kr[i] *= f[i];
}

// the same factors computed from the gate sums (readout tiles).  All 16
// lanes of a row use the same 8 tokens, so lane r of the row computes the
// factor of slot r % 8 only and a swizzle within the row (bit mode: keep
// lane bit 4, set the low bits to the slot) hands every slot to every lane.
template <int I>
__device__ __forceinline__ float row_slot(float f) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(f), 0x10 | (I << 5)));
}

__device__ __forceinline__ void gate_keys(float (&kr)[8], const float* gb, float beta_c, int ks) {
  const int lane = __lane_id(), g = lane >> 4, r = lane & 15;
  const int t = 32 * ks + 4 * g + (r & 3) + 16 * ((r >> 2) & 1);
  const float f = __builtin_amdgcn_exp2f(beta_c - gb[t]);  // both halved
  kr[0] *= row_slot<0>(f);
  kr[1] *= row_slot<1>(f);
  kr[2] *= row_slot<2>(f);
  kr[3] *= row_slot<3>(f);
  kr[4] *= row_slot<4>(f);
  kr[5] *= row_slot<5>(f);
  kr[6] *= row_slot<6>(f);
  kr[7] *= row_slot<7>(f);
}

// The value tiles only.  z is carried as the key Gram matrix Z = K^T K (the
// transposing key read is both operands) by the wave that takes tile 8 on
// the k-step, in the place of tile 8's ones-column tile (acc8[NDT - 1]).
// The key features are built from k, not sqrt(2) k: every feature, and so
// the stored value tiles, come out exactly kSpanValueScale = 1/2 of the
// state's (scaling by 2 is exact in bf16 and fp32), which saves a multiply
// per key value; the readout rescales what it loads.
template <class CF, int W, bool G = false>
__device__ __forceinline__ void state_update_dma16(f32x4 (&acc)[CF::MFT][NDT], f32x4 (&acc8)[NDT],
                                                   const DmaTile16<CF::C, G>& b, const TrOffsets& to) {
  static_assert(CF::NW == 4 && CF::NFT == 9, "d = 16 tiling");
  if constexpr (G) {
    // the chunk's decay 2^beta_C (beta at its last token)
    const float f = __builtin_amdgcn_exp2f(2.f * b.gb[CF::C - 1]);  // gb holds beta / 2
    gate_decay(acc, f);
    f32x4(&a8)[1][NDT] = *reinterpret_cast<f32x4(*)[1][NDT]>(&acc8);
    gate_decay(a8, f);
  }
#pragma unroll
  for (int ks = 0; ks < CF::C / 32; ++ks) {
    u32x4 bv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) bv[dt] = tr_operand<DV>(b.v, to.v[dt], ks);
    const u32x4 kb = tr_operand<16>(b.k, to.k, ks);
    float kr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[2 * i] = lo_bf16(kb[i]);
      kr[2 * i + 1] = hi_bf16(kb[i]);
    }
    if constexpr (G) gate_keys(kr, b.gk, ks);
    constexpr int N = NDT - 1;
    tile16_into<W, N>(acc[0], kr, bv);
    tile16_into<W + 4, N>(acc[1], kr, bv);
    if (ks % CF::NW == W) {  // compile-time per wave
      tile16_into<8, N>(acc8, kr, bv);
      if constexpr (!G) acc8[NDT - 1] = mfma(kb, kb, acc8[NDT - 1]);
    }
  }
}

// DMA instructions one wave issues per chunk
template <int C, int W, int NW, bool G = false>
constexpr int dma_count16() {
  int n = 0;
  for (int j = W; j < C / 8; j += NW) ++n;
  for (int j = W; j < C / 32; j += NW) ++n;
  if (G && (W == NW - 1 || W == NW - 2)) ++n;  // gate sums, key factors
  return n;
}

// Span layout of the d = 16 kernels.  Uniform (GL = 0): span sp covers
// chunks [sp G, (sp + 1) G).  Paired (GL > 0): spans come in pairs of 2G
// chunks, the even span of a pair GL chunks and the odd one 2G - GL, and the
// readout grid's first half takes the even spans.  With two readout
// workgroups per CU, the first half is placed first on the CUs; its waves
// are older and win the issue arbitration, so the longer spans go to them
// and both workgroups of a CU finish at about the same time.
__device__ inline int64_t span_first_chunk(const MfmaArgs& a, int64_t sp) {
  return a.GL == 0 ? sp * a.G : (sp >> 1) * 2 * a.G + ((sp & 1) ? a.GL : 0);
}

struct SpanOf {
  int64_t bh, sp;
};

__device__ inline SpanOf readout_span(const MfmaArgs& a) {
  const int64_t b = blockIdx.x;
  if (a.GL == 0) return {b / a.n_spans, b % a.n_spans};
  const int64_t per = a.n_spans / 2, half = a.BH * per;
  const int64_t odd = b >= half ? 1 : 0;
  const int64_t r = b - odd * half;
  return {r / per, 2 * (r % per) + odd};
}

// Span of a readout workgroup that adds the span sums before its span
// (a.fused).  Consecutive blocks are different heads, so with a multiple of
// 8 heads every span of a head runs on one XCD and the head's span sums,
// read by each of its later spans, stay in that XCD's L2.  The spans go
// latest first in the first half of the grid and earliest first in the
// second, so when the grid is one round of two workgroups per CU the two a
// CU receives (blocks b and b + half) add about the same number of sums
// together.
__device__ inline SpanOf fused_span(const MfmaArgs& a) {
  const int64_t b = blockIdx.x;
  const int64_t k = b / a.BH, n = a.n_spans, first = (n + 1) / 2;
  return {b % a.BH, k < first ? n - 1 - k : k - first};
}

// Span of a span-sum workgroup: spans 0 .. n_spans - 2 of every head (the
// last span's sum is never read); paired spans put the even ones first.
__device__ inline SpanOf sum_span(const MfmaArgs& a) {
  const int64_t b = blockIdx.x;
  if (a.GL == 0) return {b / (a.n_spans - 1), b % (a.n_spans - 1)};
  const int64_t per_even = a.n_spans / 2, per_odd = per_even - 1, half = a.BH * per_even;
  if (b < half) return {b / per_even, 2 * (b % per_even)};
  const int64_t r = b - half;
  return {r / per_odd, 2 * (r % per_odd) + 1};
}

// Span-state layout at d = 16 (workspace, one state per span): the value
// tiles hold kSpanValueScale times the state's value rows (the span sums
// build key features from k, not sqrt(2) k), and the z column holds the
// state's z at full scale.  The prefix sums both linearly, so the scales
// carry through it; the readout divides the value tiles by kSpanValueScale
// on load.
constexpr float kSpanValueScale = 0.5f;

// The z column of a span state from the key Gram matrix Z (lane (g, r)
// holding Z[4g + i][r]): tile J's row R gets z of the state's key features
// (weight 2 on every pair, sqrt(2) k times sqrt(2) k), 2 Z[R][R + J mod 16]
// for J = 0 .. 8, whatever scale the value tiles are stored at.  Each
// (J, R) is written by the one lane holding that entry.
template <class CF>
__device__ __forceinline__ void store_gram16(const f32x4& z, float* __restrict__ P, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i, j = (r - row) & 15;
    if (j <= 8) P[CF::ZOFF + 16 * j + row] = 2.f * z[i];
  }
}

// Three LDS buffers: chunk i is reduced while chunks i+1 and i+2 are in
// flight.  Before each chunk a wave waits for its own share of that chunk
// (vmcnt: the later chunk's transfers may stay outstanding) and the barrier
// then publishes every wave's share.  Chunks at or past the span's end read
// as zero; their reduction is skipped.
// SHORT (spans of at most four chunks, uniform layout): a fourth buffer, and
// all four chunks' transfers issued before the first reduction, so a short
// span waits for one memory latency instead of one per two chunks.
template <int C, bool G, bool SHORT = false>
__device__ __forceinline__ void span_state_dma16_body(const MfmaArgs& a) {
  using CF = Cfg<16, C>;
  constexpr int DK = 16;
  __shared__ DmaTile16<C, G> b0;
  __shared__ DmaTile16<C, G> b1;
  __shared__ DmaTile16<C, G> b2;
  __shared__ std::conditional_t<SHORT, DmaTile16<C, G>, char> b3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SpanOf span = sum_span(a);
  const int64_t bh = span.bh, sp = span.sp;
  const int64_t tok0 = bh * a.T;

  with_wave<CF::NW>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int NPC = dma_count16<C, W, CF::NW, G>();  // this wave's transfers per chunk
    f32x4 acc[CF::MFT][NDT];
    load_state<CF>(acc, nullptr, W, lane);
    f32x4 acc8[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc8[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const TrOffsets to = tr_offsets(lane);
    const int64_t first = span_first_chunk(a, sp) * C;
    int64_t end = span_first_chunk(a, sp + 1) * C;
    if (end > a.T) end = a.T;
    auto src = [&](int64_t c) { return chunk_src<DK, C>(nullptr, a.k, a.v, tok0, c, end, a.gb, a.gk); };
    dma_chunk16<C, W, CF::NW, G>(b0, src(first), lane);
    dma_chunk16<C, W, CF::NW, G>(b1, src(first + C), lane);
    if constexpr (SHORT) {
      dma_chunk16<C, W, CF::NW, G>(b2, src(first + 2 * C), lane);
      dma_chunk16<C, W, CF::NW, G>(b3, src(first + 3 * C), lane);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * NPC));
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      state_update_dma16<CF, W, G>(acc, acc8, b0, to);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * NPC));
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      if (first + C < end) state_update_dma16<CF, W, G>(acc, acc8, b1, to);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      if (first + 2 * C < end) state_update_dma16<CF, W, G>(acc, acc8, b2, to);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      if (first + 3 * C < end) state_update_dma16<CF, W, G>(acc, acc8, b3, to);
    }
    for (int64_t c0 = first; !SHORT && c0 < end; c0 += 3 * C) {
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk16<C, W, CF::NW, G>(b2, src(c0 + 2 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      state_update_dma16<CF, W, G>(acc, acc8, b0, to);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk16<C, W, CF::NW, G>(b0, src(c0 + 3 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (c0 + C < end) state_update_dma16<CF, W, G>(acc, acc8, b1, to);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk16<C, W, CF::NW, G>(b1, src(c0 + 4 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (c0 + 2 * C < end) state_update_dma16<CF, W, G>(acc, acc8, b2, to);
    }
    // drain the transfers still in flight, then add the waves' parts of tile 8
    // and of Z through LDS (4 x 64 lanes x 5 x 16 bytes = 20 KB over the tile
    // buffers)
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __syncthreads();
    constexpr int RED_BYTES = NDT * 16 * 64;  // one wave's part
    using Tile = DmaTile16<C, G>;
    static_assert(3 * sizeof(Tile) >= 4 * RED_BYTES, "reduction space");
    auto red = [&](int wv) -> f32x4* {
      if constexpr (G) {
        // gated tiles: waves 1, 2, 3 each use the start of one buffer
        static_assert(sizeof(Tile) >= RED_BYTES, "reduction space");
        return reinterpret_cast<f32x4*>(wv == 1 ? reinterpret_cast<char*>(&b0)
                                        : wv == 2 ? reinterpret_cast<char*>(&b1)
                                                  : reinterpret_cast<char*>(&b2));
      } else {
        const int off = wv * RED_BYTES;
        char* base = off < int(sizeof(Tile)) ? reinterpret_cast<char*>(&b0)
                   : off < int(2 * sizeof(Tile)) ? reinterpret_cast<char*>(&b1)
                                                 : reinterpret_cast<char*>(&b2);
        return reinterpret_cast<f32x4*>(base + off % int(sizeof(Tile)));
      }
    };
    static_assert(G || sizeof(Tile) % RED_BYTES == 0, "parts do not straddle buffers");
    if constexpr (W != 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) red(W)[dt * 64 + lane] = acc8[dt];
    }
    __syncthreads();
    if constexpr (W == 0) {
#pragma unroll
      for (int wv = 1; wv < CF::NW; ++wv) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc8[dt] += red(wv)[dt * 64 + lane];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[2][dt] = acc8[dt];
    }
    float* P = a.ws + (bh * a.n_spans + sp) * mfma_state_floats(DK);
    if constexpr (G) {
      store_state<CF>(acc, P, W, lane);  // z column: zeros (no denominator)
    } else {
      store_state<CF, false>(acc, P, W, lane);
      if constexpr (W == 0) store_gram16<CF>(acc8[NDT - 1], P, lane);
    }
  });
}

template <int C, bool G = false, bool SHORT = false>
__global__ __launch_bounds__(256) void span_state_dma16_kernel(MfmaArgs a) {
  span_state_dma16_body<C, G, SHORT>(a);
}

// ------------------------------------------------------------ readout

// per-lane constants of the readout: query and value tiles of the wave and
// the causal mask of the diagonal score tile (key 4g + j against query r)
template <class CF>
struct ReadoutLane {
  int qt[CF::NSLOT];
  int vt[CF::NDW];
  bool keep[4];
};

template <class CF>
__device__ __forceinline__ ReadoutLane<CF> readout_lane(int w, int lane) {
  ReadoutLane<CF> L;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int slot = 0; slot < CF::NSLOT; ++slot) L.qt[slot] = query_tile<CF>(w, slot);
#pragma unroll
  for (int i = 0; i < CF::NDW; ++i) L.vt[i] = value_tile<CF>(w, i);
#pragma unroll
  for (int j = 0; j < 4; ++j) L.keep[j] = 4 * g + j <= r;
  return L;
}

// Readout of one chunk by wave `w`: the chunk's queries against the state
// copy Sb (the prefix before the chunk) plus the squared causal scores of the
// chunk, normalised and stored through `dst` (rows of this chunk).
//
// The chunk's operands come from `src`: register-staged LDS tiles (TileSrc)
// or the raw tiles of the DMA path (DmaSrc16).  A source gives the fp32
// values of 4 consecutive dimensions of a query row, the score operands of a
// query / key row, and the V operand of a value tile and 32-key block.
template <class CF>
struct TileSrc {
  static constexpr bool kGramDen = false;  // denominators from the ones-column tile
  static constexpr bool kHalfDiag = false;  // Sb holds the diagonal features at full weight
  const Tiles<CF>& tl;
  __device__ __forceinline__ float4 qrow4(int row, int c4) const {
    return *reinterpret_cast<const float4*>(&tl.Qf[row * CF::QF_LD + 4 * c4]);
  }
  __device__ __forceinline__ ScoreOp<CF::FM> score_q(int row, int g) const {
    return score_operand<CF>(tl.Qf, row, g);
  }
  __device__ __forceinline__ ScoreOp<CF::FM> score_k(int row, int g) const {
    return score_operand_bf16<CF>(tl.Kb, row, g);
  }
  __device__ __forceinline__ u32x4 v_op(int vt, int s, int lane) const {
    const int g = lane >> 4, r = lane & 15;
    return *reinterpret_cast<const u32x4*>(&tl.Vt[vrow(vt, r) * CF::LDT + 32 * s + 8 * g]);
  }
};

// the register-staged tiles of the gated read: the chunk's gate row beta_t / 2
template <class CF>
struct TileSrcG : TileSrc<CF> {
  const float* gb;
  __device__ __forceinline__ float gate(int row) const { return gb[row]; }
  __device__ __forceinline__ float4 gate4(int row) const { return *reinterpret_cast<const float4*>(&gb[row]); }
};

// fp32 partial reads of a sliced feature map: rows of PART_LD floats (64
// value columns, the denominator, padding) for the chunk's tokens
constexpr int PART_LD = 68;
struct NoPart {};
struct PartRows {
  __amdgpu_buffer_rsrc_t r;
};

// `after_q` runs once the query rows are in registers (the DMA readout issues
// the next chunk's transfer there)
//
// G (gated read): the source also gives half the chunk's running gate sums,
// beta_t / 2 (log2 units).  The inter term of query t is 2^beta_t phi(q_t) S, so the
// query row is scaled by 2^(beta_t / 2); the intra score of key s is weighted
// by 2^(beta_t - beta_s); there is no denominator.
//
// Sliced maps (CF::NSL > 1): the first slice also carries the intra-chunk
// term; each slice adds its read to the fp32 partial rows `part` (the first
// writes them), and the last normalises and stores the output.
template <class CF, class S, class H = NoHook, bool G = false, class P = NoPart>
__device__ __forceinline__ void readout_chunk(const S& src, const uint16_t* __restrict__ Sb,
                                              const ReadoutLane<CF>& L, int lane, float eps,
                                              __amdgpu_buffer_rsrc_t dst, uint16_t* __restrict__ ob_tile,
                                              const H& after_q = H{}, const P& part = P{}) {
  constexpr int C = CF::C, DK = CF::DK, FM = CF::FM, NSLOT = CF::NSLOT, NDW = CF::NDW;
  constexpr int SB_LD = CF::SB_LD;
  static_assert(!G || CF::NSL == 1, "the gated read uses the full map");
  // denominators from the key Gram matrix (see below) instead of the ones-column tile
  constexpr bool ZD = S::kGramDen;
  static_assert(!ZD || (DK == 16 && NDW == NDT && !G && CF::NSL == 1), "Gram denominators: d = 16, whole rows");
  constexpr int NO = (G || ZD) ? NDW - 1 : NDW;  // value tiles read out
  constexpr int SH = Schedule<FM>::SH;
  const int g = lane >> 4, r = lane & 15;
  const int qt_max = L.qt[NSLOT - 1] > L.qt[0] ? L.qt[NSLOT - 1] : L.qt[0];

  f32x4 o[NSLOT][NDW];
  float qr[NSLOT][DK];  // this lane's query row (query 16 qt + r), rotated by g*SH
#pragma unroll
  for (int slot = 0; slot < NSLOT; ++slot) {
#pragma unroll
    for (int i = 0; i < NDW; ++i) o[slot][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DK / 4; ++c) {
      const int c4 = (c + g * (SH / 4)) % (DK / 4);
      const float4 x = src.qrow4(16 * L.qt[slot] + r, c4);
      qr[slot][4 * c + 0] = x.x;
      qr[slot][4 * c + 1] = x.y;
      qr[slot][4 * c + 2] = x.z;
      qr[slot][4 * c + 3] = x.w;
    }
  }
  float bq[NSLOT];  // gate sum of the lane's query (gated read)
  if constexpr (G) {
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      bq[slot] = src.gate(16 * L.qt[slot] + r);
      const float f = __builtin_amdgcn_exp2f(bq[slot]);  // the source holds beta / 2
#pragma unroll
      for (int c = 0; c < DK; ++c) qr[slot][c] *= f;
    }
  }
  after_q();
  // inter-chunk term.  Positions of a size-2 orbit in lane groups 2 and 3
  // and positions past the last feature hold zero state, so the query
  // feature there is left unmasked.
#pragma unroll
  for (int ks = 0; ks < CF::NKS; ++ks) {
    u32x4 bs[NDW];
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      bs[i] = *reinterpret_cast<const u32x4*>(&Sb[vrow(L.vt[i], r) * SB_LD + 32 * ks + 8 * g]);
    }
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = 8 * ks + i;
        if (e >= Schedule<FM>::NE) {
          f[i] = 0.f;
        } else {
          const int pa = kSched<FM>.a[e], pb = kSched<FM>.b[e];
          f[i] = (pa == pb && !S::kHalfDiag) ? (0.5f * qr[slot][pa]) * qr[slot][pa] : qr[slot][pa] * qr[slot][pb];
        }
      }
      const u32x4 qfeat = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
#pragma unroll
      for (int i = 0; i < NO; ++i) o[slot][i] = mfma(bs[i], qfeat, o[slot][i]);
    }
  }
  // intra-chunk term: squared causal scores.  The score product has K = d:
  // one 16x16x16 product at d = 16, one 16x16x32 product at d = 32.
  //
  // Gram denominators (ZD): the prefix part of query q's denominator is
  // phi(q) . z = q^T Z q with Z = sum_s k_s k_s^T, the 16 x 16 Gram matrix of
  // the keys before the chunk (bf16 copy from `src`).  One 16x16x16 product
  // E = Z Q^T gives lane (g, r) the entries 4g + i of Z q_r, which it dots with
  // dimensions 4g + i of q_r; the chunk part is the sum of the query's weights
  // (the bf16 values the numerator uses).  The four lane groups' shares are
  // summed at the end.
  float den[NSLOT];
#pragma unroll
  for (int slot = 0; slot < NSLOT; ++slot) den[slot] = 0.f;
  if constexpr (CF::SLICE == 0) {
  ScoreOp<FM> qf[NSLOT];
#pragma unroll
  for (int slot = 0; slot < NSLOT; ++slot) qf[slot] = src.score_q(16 * L.qt[slot] + r, g);
  if constexpr (ZD) {
    const uint2 zop = src.gram_op(r, g);
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      const f32x4 e = score_mfma<16>(zop, qf[slot]);
      float d = lo_bf16(qf[slot].x) * e[0];
      d = __builtin_fmaf(hi_bf16(qf[slot].x), e[1], d);
      d = __builtin_fmaf(lo_bf16(qf[slot].y), e[2], d);
      den[slot] = __builtin_fmaf(hi_bf16(qf[slot].y), e[3], d);
    }
  }
#pragma unroll
  for (int s = 0; s < C / 32; ++s) {
    if (2 * s > qt_max) break;
    ScoreOp<FM> kf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) kf[h] = src.score_k(16 * (2 * s + h) + r, g);
    u32x4 bv[NDW];
#pragma unroll
    for (int i = 0; i < NO; ++i) bv[i] = src.v_op(L.vt[i], s, lane);
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      if (2 * s > L.qt[slot]) continue;  // uniform per wave
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * s + h;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[h][j] = 0.f;
        if (kt > L.qt[slot]) continue;  // fully masked tile: uniform per wave
        f32x4 s2;  // squared score, [key 4g+j][query r]
        if constexpr (fm_family(FM) == 200) {
          // KATA-M2: one product per block, squares summed
          const f32x4 b0 = mfma(kf[h].p[0], qf[slot].p[0], f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 b1 = mfma(kf[h].p[1], qf[slot].p[1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < 4; ++j) s2[j] = __builtin_fmaf(b0[j], b0[j], b1[j] * b1[j]);
        } else if constexpr (kBlockMap<FM>) {
          // sum over the blocks of the squared block scores
          s2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 b = score_mfma<16>(kf[h].p[a], qf[slot].p[a]);
#pragma unroll
            for (int j = 0; j < 4; ++j) s2[j] = __builtin_fmaf(b[j], b[j], s2[j]);
          }
        } else {
          f32x4 sc;
          if constexpr (fm_family(FM) == 100) {
            // full map at d = 64: two chained 16x16x32 products
            sc = mfma(kf[h].p[0], qf[slot].p[0], f32x4{0.f, 0.f, 0.f, 0.f});
            sc = mfma(kf[h].p[1], qf[slot].p[1], sc);
          } else {
            sc = score_mfma<DK>(kf[h], qf[slot]);
          }
          if constexpr (G) {
            // p = sc^2 2^(beta_q - beta_k): fold the root of the weight,
            // 2^(beta_q / 2 - beta_k / 2), into sc
            const float4 bk = src.gate4(16 * kt + 4 * g);
            sc[0] *= __builtin_amdgcn_exp2f(bq[slot] - bk.x);
            sc[1] *= __builtin_amdgcn_exp2f(bq[slot] - bk.y);
            sc[2] *= __builtin_amdgcn_exp2f(bq[slot] - bk.z);
            sc[3] *= __builtin_amdgcn_exp2f(bq[slot] - bk.w);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) s2[j] = sc[j] * sc[j];
        }
        if (kt < L.qt[slot]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) p[h][j] = s2[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) p[h][j] = L.keep[j] ? s2[j] : 0.f;
        }
      }
      const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                        pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
      for (int i = 0; i < NO; ++i) o[slot][i] = mfma(bv[i], pf, o[slot][i]);
      if constexpr (ZD) {
#pragma unroll
        for (int i = 0; i < 4; ++i) den[slot] = dot2_bf16(pf[i], kOnesBf16x2, den[slot]);
      }
    }
  }
  if constexpr (ZD) {
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) {
      // the four 16-lane rows: swap odd and even rows, then the two halves;
      // each swap returns both registers, whose sum is the pairwise sum
      const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(den[slot]), __float_as_uint(den[slot]),
                                                        false, false);
      const float d2 = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d2), __float_as_uint(d2), false, false);
      den[slot] = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    }
  }
  }  // intra-chunk term
  if constexpr (CF::NSL > 1) {
    // partial reads: value columns 16 vt + 4g + j and (ones-column tile,
    // lanes of group 0) the denominator of query r.  With two waves sharing a
    // query tile, the one holding value tile 0 owns the denominator.
    static_assert(NDW < NDT && NSLOT == 1, "sliced maps use the 8-wave chunk-64 split");
    const bool own_den = L.vt[0] == 0 && g == 0;
    const int row = 16 * L.qt[0] + r;
    if constexpr (CF::SLICE > 0) {
      // one value tile at a time: the accumulators of the whole state are
      // live here, so the partial rows are not all loaded up front
#pragma unroll
      for (int i = 0; i < NDW; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (L.vt[i] == NDT - 1) {
          const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(part.r, (row * PART_LD + DV) * 4, 0, 0));
          if (own_den || CF::SLICE == CF::NSL - 1) o[0][i][0] += g == 0 ? x : 0.f;
        } else {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(part.r, (row * PART_LD + 16 * L.vt[i] + 4 * g) * 4, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[0][i][j] += __uint_as_float(x[j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (CF::SLICE < CF::NSL - 1) {
#pragma unroll
      for (int i = 0; i < NDW; ++i) {
        if (L.vt[i] == NDT - 1) {
          if (own_den) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[0][i][0]), part.r, (row * PART_LD + DV) * 4, 0, 0);
        } else {
          const u32x4 x = {__float_as_uint(o[0][i][0]), __float_as_uint(o[0][i][1]), __float_as_uint(o[0][i][2]),
                           __float_as_uint(o[0][i][3])};
          __builtin_amdgcn_raw_buffer_store_b128(x, part.r, (row * PART_LD + 16 * L.vt[i] + 4 * g) * 4, 0, 0);
        }
      }
      return;
    }
  }
  // normalise and store: with the ones-column tile (the last readout value
  // tile of every wave) lane r of group 0 holds the denominator of query r;
  // with Gram denominators every lane holds its query's.  Rows past T fall
  // outside `dst` and are dropped
#pragma unroll
  for (int slot = 0; slot < NSLOT; ++slot) {
    float inv = 1.f;  // the gated read has no denominator
    if constexpr (ZD) {
      inv = __builtin_amdgcn_rcpf(den[slot] + eps);
    } else if constexpr (!G) {
      const float dn = __shfl(o[slot][NDW - 1][0], r);
      inv = __builtin_amdgcn_rcpf(dn + eps);
    }
    if constexpr (CF::STAGE_OUT) {
      // whole rows: stage the 16 x 64 tile in the wave's LDS tile, then
      // write it back as 1 KB contiguous stores (16 bytes per lane)
#pragma unroll
      for (int i = 0; i < NDW - 1; ++i) {
        uint2 ob;
        ob.x = pack2(o[slot][i][0] * inv, o[slot][i][1] * inv);
        ob.y = pack2(o[slot][i][2] * inv, o[slot][i][3] * inv);
        *reinterpret_cast<uint2*>(&ob_tile[r * OB_LD + 16 * L.vt[i] + 4 * g]) = ob;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + (lane >> 3);
        const uint4 x = *reinterpret_cast<const uint4*>(&ob_tile[row * OB_LD + 8 * (lane & 7)]);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, dst,
                                               (16 * L.qt[slot] + row) * (2 * DV) + 16 * (lane & 7), 0, 0);
      }
    } else {
      const int row = 16 * L.qt[slot] + r;
#pragma unroll
      for (int i = 0; i < NDW - 1; ++i) {
        uint2 ob;
        ob.x = pack2(o[slot][i][0] * inv, o[slot][i][1] * inv);
        ob.y = pack2(o[slot][i][2] * inv, o[slot][i][3] * inv);
        buf_store8(dst, row * (2 * DV) + 2 * (16 * L.vt[i] + 4 * g), ob);
      }
    }
  }
}

// every wave reads out and carries its share of the state
// (G: the gated read -- gate row in LDS, query and score factors in the
// readout, the chunk decay and key factors in the state carry, no
// denominator)
template <class CF, bool G = false>
__device__ __forceinline__ void readout_mfma_body(const MfmaArgs& a) {
  constexpr int C = CF::C, DK = CF::DK, SB_LD = CF::SB_LD;
  __shared__ SmemOut<CF> sm;
  __shared__ alignas(16) float gbs[G ? C : 4];
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keep it scalar so every
  // wave-dependent branch is a scalar branch, not an exec-mask region
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / a.n_spans;
  const int64_t sp = blockIdx.x - bh * a.n_spans;
  const int64_t tok0 = bh * a.T;

  // feature positions no tile writes hold no feature: zero once
  for (int e = tid; e < VROWS * CF::NPOS; e += CF::NT) {
    const int c = e % CF::NPOS;
    if (sb_col_unused<CF>(c)) sm.Sb[(e / CF::NPOS) * SB_LD + c] = 0;
  }
  init_const_rows<CF>(sm, tid);
  with_wave<CF::NW>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const KeyPairs<CF> kp = key_pairs<CF>(W, lane & 15);
    const ReadoutLane<CF> L = readout_lane<CF>(W, lane);
    f32x4 acc[CF::MFT][NDT];
    load_state<CF>(acc, a.n_spans > 1 ? a.ws + (bh * a.n_spans + sp) * mfma_state_floats(DK) : nullptr,
                   W, lane);
    write_sb<CF>(sm.Sb, acc, W, lane);
    // An unconditional vmcnt(0) retires the state loads for the wait-count
    // analysis, which would otherwise keep them pending into the chunk loop
    // and stall its MFMAs on the in-order count of the chunk prefetches.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // chunk i is read from LDS while chunk i+1 arrives in registers; after
    // the chunk's reads a single phase writes the next state copy and stages
    // the next chunk (disjoint LDS regions), so each chunk costs two barriers
    Stage<CF, true, G> st;
    const int64_t first = sp * a.G * C;
    int64_t end = first + a.G * C;
    if (end > a.T) end = a.T;
    auto src = [&](int64_t c) { return chunk_src<DK, C>(a.q, a.k, a.v, tok0, c, a.T, a.gb, a.gk); };
    st.load(src(first), tid);
    st.store(sm, tid, gbs);
    __syncthreads();
    for (int64_t c0 = first; c0 < end; c0 += C) {
      // the next chunk's loads go out first, to overlap this chunk's compute
      if (c0 + C < end) st.load(src(c0 + C), tid);
      const int64_t n = (a.T - c0 < C) ? a.T - c0 : C;
      if constexpr (G) {
        readout_chunk<CF, TileSrcG<CF>, NoHook, true>(TileSrcG<CF>{{sm}, gbs}, sm.Sb, L, lane, a.eps,
                                                      rows_rsrc(a.out, tok0 + c0, n, 2 * DV),
                                                      sm.Ob[CF::NDW == NDT ? W : 0]);
      } else if constexpr (CF::NSL > 1) {
        readout_chunk<CF, TileSrc<CF>, NoHook, false, PartRows>(
            TileSrc<CF>{sm}, sm.Sb, L, lane, a.eps, rows_rsrc(a.out, tok0 + c0, n, 2 * DV), sm.Ob[0], NoHook{},
            PartRows{rows_rsrc(a.part, tok0 + c0, n, PART_LD * 4)});
      } else {
        readout_chunk<CF>(TileSrc<CF>{sm}, sm.Sb, L, lane, a.eps, rows_rsrc(a.out, tok0 + c0, n, 2 * DV),
                          sm.Ob[CF::NDW == NDT ? W : 0]);
      }
      if (c0 + C >= end) break;
      // carry the state across the chunk
      if constexpr (G) {
        gate_decay(acc, __builtin_amdgcn_exp2f(2.f * gbs[C - 1]));  // a whole chunk: beta_C / 2
        state_update<CF, SmemOut<CF>, NDT - 1>(acc, sm, W, lane, kp);
      } else {
        state_update<CF>(acc, sm, W, lane, kp);
      }
      __syncthreads();  // every wave done reading the tiles and Sb of this chunk
      write_sb<CF>(sm.Sb, acc, W, lane);
      st.store(sm, tid, gbs);
      __syncthreads();
    }
  });
}

template <class CF, bool G = false>
__global__ __launch_bounds__(CF::NT, 2) void readout_mfma_kernel(MfmaArgs a) {
  readout_mfma_body<CF, G>(a);
}

// ------------------------------------------------------------ readout, d = 32, wave-specialised
//
// The d = 32 chunked readout at chunk 64 with the 8 waves split by role.
// Waves 0..3 read out one query tile each (all four value tiles): the inter
// term phi_q(Q_c) S from the state copy and the prefix denominator.  Waves
// 4..7 carry the state across the chunk (state wave u owns feature tiles
// u, u + 4, ..., u + 32 of the 33) and form the squared causal block of one
// query tile each, which they hand to its readout wave through LDS; so every
// query feature and every key feature is built exactly once per chunk.  Per
// chunk the readout waves run the inter term while the state waves run the
// intra-chunk blocks and the state update; after the barrier the readout
// waves add the block, normalise and store while the state waves publish the
// new state copy.  The denominators take the key Gram matrix
// Z = sum_s k_s k_s^T (32 x 32, on state wave 3, one product per 16 x 16 tile
// and 32 keys from the transposing read of the bf16 K rows): phi_q(q) . z =
// q^T Z q, from two 16x16x32 products E = Z Q^T per query tile and a dot with
// q; the chunk part is the vector sum of the query's bf16 weights.  No
// ones-column tile.  Feature positions follow the rotation schedule below:
// the transposing read gives lane (g, R) dimensions R and 16 + R of its 8
// tokens, and every key feature is one multiply of one of them by one of
// lane R + j's, the rotation folded in.  No fp32 K copy.  The key features
// carry weight 1 (the products of bf16 k are exact), so the state waves hold
// half the state (halved on load) and the state copy is read with query
// features of weight 1 on the diagonal and 2 off it.  The readout waves stage
// the chunk (V transposed, Q as fp32 rows, the bf16 K rows); the state waves
// stage the gate sums of the gated read.  The span state in the workspace
// holds the value tiles at full scale and the z column as 2 Z[a][b] on the
// position of the pair (a, b), the sum of the key features.
using CfgWs32 = Cfg<32, 64, 8>;   // tiles and strides
constexpr int ZB_LD = 40;         // bf16 row stride of the Gram copy

// The feature schedule of the wave-specialised d = 32 kernels (17 k-steps of
// 32 positions, feature tile ft = 2 ks + h, row R = position 32 ks + 16 h + R).
// Every tile is a row rotation: row R holds the pair (R + 16 h1,
// (R + j) mod 16 + 16 h2), which the key side builds as x_h1 times x_h2 of
// lane R + j of its 16-lane row (x0, x1: dimensions r and 16 + r of the
// lane's tokens), one multiply with the rotation folded in and no select:
//   ks = 0..7,  j = ks:     h = 0: (0, 0, j)   h = 1: (1, 1, j)   pairs inside each half
//   ks = 8..14, j = ks - 7: h = 0: (0, 1, j)   h = 1: (1, 0, j)   cross pairs at offsets j, 16 - j
//   ks = 15:                h = 0: (0, 1, 0)   h = 1: (0, 1, 8)   cross pairs at offsets 0, 8
//   ks = 16:                h = 0: rows 0..7 (R, R + 8) and rows 8..15 (R + 8, R + 16)
//                           (offset 8 inside each half); h = 1 holds nothing.
// The query side: lane group g holds positions 8 g + i of each k-step, the
// pair (pi_g(A), pi_g(B)) of a compile-time pattern (A, B) of entry i, where
// pi_g exchanges the halves of the dimensions for g >= 2 and rotates each
// half by 8 for odd g.  The lane reads its query row permuted by pi_g once
// per chunk and indexes it at compile time; k-steps 15 and 16 take a second
// pattern on lane groups 2 and 3 (k-step 15) or 1 (k-step 16), and k-step
// 16 nothing on groups 2 and 3.
struct Ws32Pair {
  int a, b;
};
__host__ __device__ constexpr int ws32_pi(int dim, int g) {
  return 16 * ((dim >> 4) ^ (g >> 1)) + (((dim & 15) + 8 * (g & 1)) & 15);
}
// pattern of entry i of k-step ks (alt: the second pattern)
__host__ __device__ constexpr Ws32Pair ws32_pattern(int ks, bool alt, int i) {
  if (ks < 8) return {i, (i + ks) & 15};
  if (ks < 15) return {i, 16 + ((i + ks - 7) & 15)};
  if (ks == 15) return alt ? Ws32Pair{16 + i, 8 + i} : Ws32Pair{i, 16 + i};
  return alt ? Ws32Pair{24 + i, 16 + i} : Ws32Pair{i, 8 + i};
}
// the pattern lane group g of k-step ks uses: 0, 1 (the second) or -1 (none)
__host__ __device__ constexpr int ws32_variant(int ks, int g) {
  if (ks < 15) return 0;
  if (ks == 15) return g >= 2 ? 1 : 0;
  return g == 0 ? 0 : g == 1 ? 1 : -1;
}
// the pair the query side places at feature position p (a < 0: none)
constexpr Ws32Pair ws32_pair_at(int p) {
  const int ks = p >> 5, g = (p >> 3) & 3, i = p & 7;
  const int var = ks < 17 ? ws32_variant(ks, g) : -1;
  if (var < 0) return {-1, -1};
  const Ws32Pair e = ws32_pattern(ks, var == 1, i);
  return {ws32_pi(e.a, g), ws32_pi(e.b, g)};
}
// key tile ft: row R pairs R + 16 h1 with (R + j) mod 16 + 16 h2; h1 < 0 for
// the mixed tile 32, h1 = -2 for the empty tile 33
struct Ws32Key {
  int h1, h2, j;
};
constexpr Ws32Key ws32_key(int ft) {
  const int ks = ft >> 1, h = ft & 1;
  if (ks < 8) return {h, h, ks};
  if (ks < 15) return {h, 1 - h, ks - 7};
  if (ks == 15) return {0, 1, h ? 8 : 0};
  return {h ? -2 : -1, 0, 8};
}
// both sides place the same pair on every position, and every pair a <= b
// has exactly one position
constexpr bool ws32_schedule_ok() {
  bool seen[32][32] = {};
  int n = 0;
  for (int p = 0; p < 17 * 32; ++p) {
    const Ws32Pair q = ws32_pair_at(p);
    const int R = p & 15;
    const Ws32Key k = ws32_key(p >> 4);
    int ka = -1, kb = -1;
    if (k.h1 == -1) {
      ka = R < 8 ? R : 16 + R;
      kb = R < 8 ? R + 8 : R + 8;
    } else if (k.h1 >= 0) {
      ka = R + 16 * k.h1;
      kb = ((R + k.j) & 15) + 16 * k.h2;
    }
    if ((q.a < 0) != (ka < 0)) return false;
    if (q.a < 0) continue;
    if (!((q.a == ka && q.b == kb) || (q.a == kb && q.b == ka))) return false;
    const int x = q.a < q.b ? q.a : q.b, y = q.a < q.b ? q.b : q.a;
    if (seen[x][y]) return false;
    seen[x][y] = true;
    ++n;
  }
  return n == 32 * 33 / 2;
}
static_assert(ws32_schedule_ok(), "the wave-specialised d = 32 schedule covers every pair once");
static_assert(Schedule<32>::NKS == 17, "the wave-specialised d = 32 kernels use 17 k-steps");

// feature position of every pair (a, b) of that schedule (symmetric)
struct PairPos32 {
  int16_t p[32][32];
};
constexpr PairPos32 make_pair_pos32() {
  PairPos32 t{};
  for (int a = 0; a < 32; ++a)
    for (int b = 0; b < 32; ++b) t.p[a][b] = -1;
  for (int p = 0; p < 17 * 32; ++p) {
    const Ws32Pair q = ws32_pair_at(p);
    if (q.a < 0) continue;
    t.p[q.a][q.b] = static_cast<int16_t>(p);
    t.p[q.b][q.a] = static_cast<int16_t>(p);
  }
  return t;
}
constexpr bool pair_pos32_ok() {
  constexpr PairPos32 t = make_pair_pos32();
  for (int a = 0; a < 32; ++a)
    for (int b = 0; b < 32; ++b)
      if (t.p[a][b] < 0 || t.p[a][b] >= 16 * mfma_feature_tiles(32)) return false;
  return true;
}
static_assert(pair_pos32_ok(), "every d = 32 pair has a feature position");
__constant__ PairPos32 kPairPos32 = make_pair_pos32();

// The bf16 state copy in the order the inter-term products read it: for
// k-step j and value tile i, the 64 lanes' 16-byte A operands (lane (g, r):
// value row 16 i + r, feature positions 32 j + 8 g .. + 7) lie contiguous,
// so each operand read is one contiguous 1 KB.
constexpr int kSbo32Elems = Schedule<32>::NKS * (NDT - 1) * 64 * 8;
__device__ __forceinline__ int sbo32(int ks, int vt, int lane) { return ((ks * (NDT - 1) + vt) * 64 + lane) * 8; }

struct alignas(16) SmemWs32 : Tiles<CfgWs32> {
  alignas(16) uint16_t Sb[kSbo32Elems];   // bf16 state copy, operand order
  alignas(16) uint16_t Zb[32 * ZB_LD];    // bf16 Gram matrix, row-major
  alignas(16) uint16_t Ob[4][16 * OB_LD]; // per readout wave output tile
  alignas(16) float gbs[64];              // gated read: beta_t / 2 of the chunk
  alignas(16) float gks[64];              // gated read: key factors 2^((beta_C - beta_t) / 2)
  // the intra-chunk term of each query tile, from the state waves to the
  // readout waves: the four fp32 accumulator tiles in lane order, and each
  // lane's part of the denominator
  alignas(16) float Xo[4][(NDT - 1) * 64 * 4];
  alignas(16) float Xd[4][64];
};
static_assert(sizeof(SmemWs32) <= 160 * 1024, "the d = 32 readout's LDS fits one CU");

// Staging of one chunk by the readout waves (threads 0..255): V (transposed),
// Q (fp32 rows) and the bf16 K rows; the state waves stage nothing.  Tokens
// at or past the end read as zero.
struct StageWs32 {
  static constexpr int C = 64, DK = 32;
  uint4 x[4];  // V: 4 tokens x 16 bytes; Q or K: one 64-byte row

  __device__ __forceinline__ void load(const ChunkSrc& src, int tid) {
    if (tid < 128) {  // V: token group tid % 16, column group tid / 16
      const int tg = tid % (C / 4), cg = tid / (C / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = buf_load16(src.v, (4 * tg + r) * (2 * DV) + 16 * cg);
    } else if (tid < 192) {  // Q row
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = buf_load16(src.q, (tid - 128) * (2 * DK) + 16 * u);
    } else if (tid < 256) {  // K row
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = buf_load16(src.k, (tid - 192) * (2 * DK) + 16 * u);
    }
  }

  __device__ __forceinline__ void store(SmemWs32& sm, int tid) const {
    using CF = CfgWs32;
    if (tid < 128) {
      const int tg = tid % (C / 4), cg = tid / (C / 4);
      const int pos = group_pos(tg);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int w = c >> 1;
        const uint32_t w0 = w == 0 ? x[0].x : w == 1 ? x[0].y : w == 2 ? x[0].z : x[0].w;
        const uint32_t w1 = w == 0 ? x[1].x : w == 1 ? x[1].y : w == 2 ? x[1].z : x[1].w;
        const uint32_t w2 = w == 0 ? x[2].x : w == 1 ? x[2].y : w == 2 ? x[2].z : x[2].w;
        const uint32_t w3 = w == 0 ? x[3].x : w == 1 ? x[3].y : w == 2 ? x[3].z : x[3].w;
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint2 o;
        o.x = __builtin_amdgcn_perm(w1, w0, sel);
        o.y = __builtin_amdgcn_perm(w3, w2, sel);
        *reinterpret_cast<uint2*>(&sm.Vt[(8 * cg + c) * CF::LDT + pos]) = o;
      }
    } else if (tid < 192) {
      const int t = tid - 128;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float4 f;
          f.x = lo_bf16(v[2 * h]);
          f.y = hi_bf16(v[2 * h]);
          f.z = lo_bf16(v[2 * h + 1]);
          f.w = hi_bf16(v[2 * h + 1]);
          *reinterpret_cast<float4*>(&sm.Qf[t * CF::QF_LD + 8 * u + 4 * h]) = f;
        }
      }
    } else if (tid < 256) {
      const int t = tid - 192;
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(&sm.Kb[t * CF::KB_LD + 8 * u]) = x[u];
    }
  }
};

// Gated read: the chunk's gate sums (state-wave threads u = 0..15) and key
// factors (u = 16..31), 16 bytes each, staged by the state waves (whose
// registers have room; the readout waves' have none).
struct GateStageWs32 {
  uint4 x;
  __device__ __forceinline__ void load(const ChunkSrc& src, int u) {
    if (u < 16) {
      x = buf_load16(src.g, 16 * u);
    } else if (u < 32) {
      x = buf_load16(src.gk, 16 * (u - 16));
    }
  }
  __device__ __forceinline__ void store(SmemWs32& sm, int u) const {
    if (u < 16) {
      *reinterpret_cast<uint4*>(&sm.gbs[4 * u]) = x;
    } else if (u < 32) {
      *reinterpret_cast<uint4*>(&sm.gks[4 * (u - 16)]) = x;
    }
  }
};

// transposing read of the bf16 K rows for the Gram matrix: lane (g, s) gets
// dimension 16 I + s of the 8 tokens 32 ks + 4g + m, 32 ks + 16 + 4g + m
__device__ __forceinline__ u32x4 gram_operand32(const uint16_t* Kb, int I, int ks, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int off = (4 * g + (s >> 2)) * CfgWs32::KB_LD + 16 * I + 4 * (s & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint2 v = tr_read(&Kb[off + (32 * ks + 16 * h) * CfgWs32::KB_LD]);
    out[2 * h] = v.x;
    out[2 * h + 1] = v.y;
  }
  return out;
}

// feature tile ft of the wave-specialised d = 32 schedule for the lane's 8
// tokens: row R (= lane r of the row) takes x_h1 times x_h2 of lane
// (R + j) mod 16; tile 32 takes offset 8 inside the first half on rows 0..7
// and inside the second on rows 8..15 (weight 1 on every pair: the state
// waves keep half the state)
template <int FT>
__device__ __forceinline__ void ws32_key_tile(f32x4 (&acc)[NDT - 1], const float (&x)[2][8],
                                              const u32x4 (&bv)[NDT - 1], int r) {
  constexpr Ws32Key K = ws32_key(FT);
  static_assert(K.h1 != -2, "tile 33 holds no feature");
  float f[8];
  if constexpr (K.h1 < 0) {
    const bool lo = r < 8;
    float f0[8], f1[8];
    mul_row_rotated<8>(f0, x[0], x[0]);
    mul_row_rotated<8>(f1, x[1], x[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = lo ? f0[i] : f1[i];
  } else if constexpr (K.j == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = x[K.h1][i] * x[K.h2][i];
  } else {
    mul_row_rotated<K.j>(f, x[K.h1], x[K.h2]);
  }
  const u32x4 af = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
#pragma unroll
  for (int dt = 0; dt < NDT - 1; ++dt) acc[dt] = mfma(af, bv[dt], acc[dt]);
}

// the feature tiles U, U + STRIDE, ... of one wave
template <int U, int STRIDE = 4, int MT, int... M>
__device__ __forceinline__ void ws32_key_tiles(f32x4 (&acc)[MT][NDT - 1], const float (&x)[2][8],
                                               const u32x4 (&bv)[NDT - 1], int r,
                                               std::integer_sequence<int, M...>) {
  (ws32_key_tile<U + STRIDE * M>(acc[M], x, bv, r), ...);
}

// gated read: the key factors 2^((beta_C - beta_t) / 2) of the lane's 8
// tokens (32 ks + 4 g + m and 32 ks + 16 + 4 g + m) on both halves' values
__device__ __forceinline__ void ws32_gate_keys(float (&x)[2][8], const float* gk, int ks, int g) {
  const float4 f0 = *reinterpret_cast<const float4*>(&gk[32 * ks + 4 * g]);
  const float4 f1 = *reinterpret_cast<const float4*>(&gk[32 * ks + 16 + 4 * g]);
  const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[0][i] *= f[i];
    x[1][i] *= f[i];
  }
}

// state wave U: the feature tiles it owns, whether it keeps the key Gram
// matrix, and the query tile whose intra-chunk term it forms (the heavier
// blocks, 11 and 12 products, on the waves with 8 tiles and no Gram matrix;
// 5 and 6 products on the waves with 72 state products)
template <int U>
struct Ws32State {
  static constexpr int MT = (mfma_feature_tiles(32) - U + 3) / 4;  // feature tiles owned
  static constexpr bool GRAM = U == 3;
  static constexpr int QI = U == 0 ? 0 : U == 1 ? 3 : U == 2 ? 2 : 1;
};

// G: the gated read (GatedKATA).  The readout waves scale the query row by
// 2^(beta_q / 2) (the inter term carries 2^beta_q), weight each squared score
// by 2^(beta_q - beta_k) and keep no denominator; the state waves decay the
// state by 2^beta_C per chunk and scale the keys by 2^((beta_C - beta_t) / 2);
// there is no Gram matrix.
// FP (a.fused): the span sums are stored unscanned and the state waves add
// those of the spans before this one in span order (blocks mapped to spans
// by head first, as for the d = 16 readout).
template <bool G = false, bool FP = false>
__device__ __forceinline__ void readout_ws32(const MfmaArgs& a) {
  static_assert(!(G && FP), "the gated read takes its prefix from the affine scan");
  using CF = CfgWs32;
  constexpr int C = 64, DK = 32, NT = 512;
  __shared__ SmemWs32 sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SpanOf span = FP ? fused_span(a) : SpanOf{blockIdx.x / a.n_spans, blockIdx.x % a.n_spans};
  const int64_t bh = span.bh, sp = span.sp;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * C;
  int64_t end = first + a.G * C;
  if (end > a.T) end = a.T;
  const float* prefix =
      (!FP && a.n_spans > 1) ? a.ws + (bh * a.n_spans + sp) * mfma_state_floats(DK) : nullptr;
  // FP: the head's span sums, sp of them before this span
  const float* sums = FP ? a.ws + bh * a.n_spans * mfma_state_floats(DK) : nullptr;

  // feature positions no tile writes hold no feature (tile 33: lane groups
  // 2 and 3 of the last k-step): zero once
  for (int e = tid; e < (NDT - 1) * 32 * 8; e += NT) {
    const int vt = e / 256, l = 32 + (e / 8) % 32, j = e % 8;
    sm.Sb[sbo32(Schedule<32>::NKS - 1, vt, l) + j] = 0;
  }

  auto src = [&](int64_t c) { return chunk_src<DK, C>(a.q, a.k, a.v, tok0, c, a.T, a.gb, a.gk); };

  with_wave<8>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    if constexpr (W < 4) {
      StageWs32 st;
      st.load(src(first), tid);
      // ---------------------------------------------------------------- readout wave
      constexpr int QT = W;
      st.store(sm, tid);
      __syncthreads();  // state copy, Gram copy and chunk 0 in place
      for (int64_t c0 = first; c0 < end; c0 += C) {
        const bool more = c0 + C < end;
        if (more) st.load(src(c0 + C), tid);
        const int64_t n = (a.T - c0 < C) ? a.T - c0 : C;
        // the query row permuted by pi_g (the lane group's share of the pairs):
        // 4-dimension block c holds block pi_g(4 c) / 4 of the row
        float qr[DK];
#pragma unroll
        for (int c = 0; c < DK / 4; ++c) {
          const int blk = ((c & 4) ^ (4 * (g >> 1))) | ((c + 2 * (g & 1)) & 3);
          const float4 x = *reinterpret_cast<const float4*>(&sm.Qf[(16 * QT + r) * CF::QF_LD + 4 * blk]);
          qr[4 * c + 0] = x.x;
          qr[4 * c + 1] = x.y;
          qr[4 * c + 2] = x.z;
          qr[4 * c + 3] = x.w;
        }
        if constexpr (G) {
          // beta_q / 2 of the query into its row
          const float f = __builtin_amdgcn_exp2f(sm.gbs[16 * QT + r]);
#pragma unroll
          for (int c = 0; c < DK; ++c) qr[c] *= f;
        }
        f32x4 o[NDT - 1];
#pragma unroll
        for (int i = 0; i < NDT - 1; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        // inter term phi_q(Q_c) S against the state copy, which holds half the
        // state: query features at weight 1 on the diagonal and 2 off it
        float qr2[DK];
#pragma unroll
        for (int c = 0; c < DK; ++c) qr2[c] = 2.f * qr[c];
#pragma unroll
        for (int ks = 0; ks < Schedule<32>::NKS; ++ks) {
          u32x4 bs[NDT - 1];
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) bs[i] = *reinterpret_cast<const u32x4*>(&sm.Sb[sbo32(ks, i, lane)]);
          float f[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            constexpr auto feat = [](const float* q, const float* q2, Ws32Pair e) {
              return e.a == e.b ? q[e.a] * q[e.a] : q2[e.a] * q[e.b];
            };
            const float f0 = feat(qr, qr2, ws32_pattern(ks, false, i));
            if (ks < 15) {
              f[i] = f0;
            } else {
              const float f1 = feat(qr, qr2, ws32_pattern(ks, true, i));
              f[i] = ks == 15 ? (g >= 2 ? f1 : f0) : (g == 0 ? f0 : g == 1 ? f1 : 0.f);
            }
          }
          const u32x4 qfeat = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) o[i] = mfma(bs[i], qfeat, o[i]);
        }
        // prefix denominator q^T Z q: E = Z Q^T (two products), dotted with q
        float den = 0.f;
        if constexpr (!G) {
          const u32x4 qf = score_operand<CF>(sm.Qf, 16 * QT + r, g);
#pragma unroll
          for (int I = 0; I < 2; ++I) {
            const u32x4 zr = *reinterpret_cast<const u32x4*>(&sm.Zb[(16 * I + r) * ZB_LD + 8 * g]);
            const f32x4 e4 = mfma(zr, qf, f32x4{0.f, 0.f, 0.f, 0.f});
            const float4 qa = *reinterpret_cast<const float4*>(&sm.Qf[(16 * QT + r) * CF::QF_LD + 16 * I + 4 * g]);
            den = __builtin_fmaf(qa.x, e4[0], den);
            den = __builtin_fmaf(qa.y, e4[1], den);
            den = __builtin_fmaf(qa.z, e4[2], den);
            den = __builtin_fmaf(qa.w, e4[3], den);
          }
        }
        __syncthreads();  // intra-chunk terms in place; every wave done with the chunk, Sb and Zb
        // the intra-chunk term a state wave formed for this query tile (same
        // lane layout as o)
#pragma unroll
        for (int i = 0; i < NDT - 1; ++i) o[i] += *reinterpret_cast<const f32x4*>(&sm.Xo[QT][(64 * i + lane) * 4]);
        float inv = 1.f;  // the gated read has no denominator
        if constexpr (!G) {
          den += sm.Xd[QT][lane];
          // the four 16-lane rows hold parts of the query's denominator
          const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(den), __float_as_uint(den), false, false);
          const float d2 = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
          const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d2), __float_as_uint(d2), false, false);
          den = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
          inv = __builtin_amdgcn_rcpf(den + a.eps);
        }
        uint16_t* ob = sm.Ob[W];
#pragma unroll
        for (int i = 0; i < NDT - 1; ++i) {
          uint2 x;
          x.x = pack2(o[i][0] * inv, o[i][1] * inv);
          x.y = pack2(o[i][2] * inv, o[i][3] * inv);
          *reinterpret_cast<uint2*>(&ob[r * OB_LD + 16 * i + 4 * g]) = x;
        }
        const __amdgpu_buffer_rsrc_t dst = rows_rsrc(a.out, tok0 + c0, n, 2 * DV);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 8 * h + (lane >> 3);
          const uint4 x = *reinterpret_cast<const uint4*>(&ob[row * OB_LD + 8 * (lane & 7)]);
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, dst,
                                                 (16 * QT + row) * (2 * DV) + 16 * (lane & 7), 0, 0);
        }
        if (more) st.store(sm, tid);
        __syncthreads();  // next chunk, state copy and Gram copy in place
      }
    } else {
      // ---------------------------------------------------------------- state wave
      constexpr int U = W - 4;
      constexpr int MT = Ws32State<U>::MT;
      constexpr bool GRAM = Ws32State<U>::GRAM && !G;
      constexpr int QI = Ws32State<U>::QI;
      bool keep[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) keep[j] = 4 * g + j <= r;
      f32x4 acc[MT][NDT - 1];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int ft = U + 4 * m;
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt) {
          acc[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (prefix != nullptr) {
            // the state waves keep half the state (key features at weight 1)
            const float4 x = *reinterpret_cast<const float4*>(prefix + ((ft * (NDT - 1) + dt) * 64 + lane) * 4);
            acc[m][dt] = 0.5f * f32x4{x.x, x.y, x.z, x.w};
          }
        }
      }
      if constexpr (FP) {
        // the prefix the sequential pass would form, summed in span order
#pragma unroll 2
        for (int64_t s = 0; s < sp; ++s) {
          const float* P = sums + s * mfma_state_floats(DK);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int ft = U + 4 * m;
#pragma unroll
            for (int dt = 0; dt < NDT - 1; ++dt) {
              const float4 x = *reinterpret_cast<const float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4);
              acc[m][dt] += f32x4{x.x, x.y, x.z, x.w};
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int dt = 0; dt < NDT - 1; ++dt) acc[m][dt] *= 0.5f;
        }
      }
      // Gram tiles (I, J): lane (g, r) holds Z[16 I + 4 g + i][16 J + r]; from
      // the prefix's z column, 2 Z[a][b] on the position of (a, b)
      f32x4 zt[GRAM ? 4 : 1];
      if constexpr (GRAM) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int I = t >> 1, J = t & 1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ra = 16 * I + 4 * g + i, cb = 16 * J + r;
            const int off = CF::ZOFF + kPairPos32.p[ra][cb];
            if constexpr (FP) {
              float z = 0.f;
              for (int64_t s = 0; s < sp; ++s) z += sums[s * mfma_state_floats(DK) + off];
              zt[t][i] = 0.5f * z;
            } else {
              zt[t][i] = prefix != nullptr ? 0.5f * prefix[off] : 0.f;
            }
          }
        }
      }
      // the state copy of the owned tiles, and the Gram copy
      auto publish = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int ft = U + 4 * m;
#pragma unroll
          for (int dt = 0; dt < NDT - 1; ++dt) {
            uint2 x;
            x.x = pack2(acc[m][dt][0], acc[m][dt][1]);
            x.y = pack2(acc[m][dt][2], acc[m][dt][3]);
            // positions 32 j + 16 h + 4 g .. + 3 of value row 16 dt + r: half
            // g & 1 of the operand of lane (2 h + g / 2, r)
            *reinterpret_cast<uint2*>(&sm.Sb[sbo32(ft >> 1, dt, 16 * (2 * (ft & 1) + (g >> 1)) + r) + 4 * (g & 1)]) = x;
          }
        }
        if constexpr (GRAM) {
          // Z is symmetric: lane (g, r) writes row 16 J + r, columns 16 I + 4 g ..
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int I = t >> 1, J = t & 1;
            *reinterpret_cast<uint2*>(&sm.Zb[(16 * J + r) * ZB_LD + 16 * I + 4 * g]) =
                make_uint2(pack2(zt[t][0], zt[t][1]), pack2(zt[t][2], zt[t][3]));
          }
        }
      };
      GateStageWs32 gs;
      if constexpr (G) {
        gs.load(src(first), tid - 256);
        gs.store(sm, tid - 256);
      }
      publish();
      __syncthreads();  // state copy, Gram copy and chunk 0 in place
      for (int64_t c0 = first; c0 < end; c0 += C) {
        const bool more = c0 + C < end;
        if constexpr (G) {
          if (more) gs.load(src(c0 + C), tid - 256);
        }
        {
          // intra-chunk term of query tile QI: squared causal scores times V,
          // and (ungated) each lane's part of their sum, for the readout wave
          // of that tile
          const u32x4 qf = score_operand<CF>(sm.Qf, 16 * QI + r, g);
          float bq = 0.f;  // gated read: beta_q / 2
          if constexpr (G) bq = sm.gbs[16 * QI + r];
          f32x4 o[NDT - 1];
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          float den = 0.f;
#pragma unroll
          for (int s = 0; s <= QI / 2; ++s) {
            float p[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int kt = 2 * s + h;
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = 0.f;
              if (kt > QI) continue;
              const u32x4 kf = *reinterpret_cast<const u32x4*>(&sm.Kb[(16 * kt + r) * CF::KB_LD + 8 * g]);
              f32x4 sc = mfma(kf, qf, f32x4{0.f, 0.f, 0.f, 0.f});
              if constexpr (G) {
                // p = sc^2 2^(beta_q - beta_k): the root of the weight into sc
                const float4 bk = *reinterpret_cast<const float4*>(&sm.gbs[16 * kt + 4 * g]);
                sc[0] *= __builtin_amdgcn_exp2f(bq - bk.x);
                sc[1] *= __builtin_amdgcn_exp2f(bq - bk.y);
                sc[2] *= __builtin_amdgcn_exp2f(bq - bk.z);
                sc[3] *= __builtin_amdgcn_exp2f(bq - bk.w);
              }
#pragma unroll
              for (int j = 0; j < 4; ++j) p[h][j] = (kt < QI || keep[j]) ? sc[j] * sc[j] : 0.f;
            }
            const u32x4 pf = {pack2(p[0][0], p[0][1]), pack2(p[0][2], p[0][3]),
                              pack2(p[1][0], p[1][1]), pack2(p[1][2], p[1][3])};
#pragma unroll
            for (int i = 0; i < NDT - 1; ++i) {
              const u32x4 bv = *reinterpret_cast<const u32x4*>(&sm.Vt[(16 * i + r) * CF::LDT + 32 * s + 8 * g]);
              o[i] = mfma(bv, pf, o[i]);
            }
            if constexpr (!G) {
#pragma unroll
              for (int i = 0; i < 4; ++i) den = dot2_bf16(pf[i], kOnesBf16x2, den);
            }
          }
#pragma unroll
          for (int i = 0; i < NDT - 1; ++i) *reinterpret_cast<f32x4*>(&sm.Xo[QI][(64 * i + lane) * 4]) = o[i];
          if constexpr (!G) sm.Xd[QI][lane] = den;
        }
        if (more) {
          // carry the state across the chunk: phi_k(K_c)^T V_c and K_c^T K_c
          // (gated: the state decays by 2^beta_C first)
          if constexpr (G) {
            const float f = __builtin_amdgcn_exp2f(2.f * sm.gbs[C - 1]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
              for (int dt = 0; dt < NDT - 1; ++dt) acc[m][dt] *= f;
            }
          }
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks) {
            u32x4 bv[NDT - 1];
#pragma unroll
            for (int dt = 0; dt < NDT - 1; ++dt) {
              bv[dt] = *reinterpret_cast<const u32x4*>(&sm.Vt[(16 * dt + r) * CF::LDT + 32 * ks + 8 * g]);
            }
            // dimensions r and 16 + r of the lane's 8 tokens
            const u32x4 k0 = gram_operand32(sm.Kb, 0, ks, lane);
            const u32x4 k1 = gram_operand32(sm.Kb, 1, ks, lane);
            if constexpr (GRAM) {
              zt[0] = mfma(k0, k0, zt[0]);
              zt[1] = mfma(k0, k1, zt[1]);
              zt[2] = mfma(k1, k0, zt[2]);
              zt[3] = mfma(k1, k1, zt[3]);
            }
            float x[2][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[0][2 * i] = lo_bf16(k0[i]);
              x[0][2 * i + 1] = hi_bf16(k0[i]);
              x[1][2 * i] = lo_bf16(k1[i]);
              x[1][2 * i + 1] = hi_bf16(k1[i]);
            }
            if constexpr (G) ws32_gate_keys(x, sm.gks, ks, g);
            ws32_key_tiles<U>(acc, x, bv, r, std::make_integer_sequence<int, MT>{});
          }
        }
        __syncthreads();  // intra-chunk terms in place; every wave done with the chunk, Sb and Zb
        if (more) {
          publish();
          if constexpr (G) gs.store(sm, tid - 256);
        }
        __syncthreads();  // next chunk, state copy and Gram copy in place
      }
    }
  });
}

template <bool G = false, bool FP = false>
__global__ __launch_bounds__(512, 2) void readout_ws32_kernel(MfmaArgs a) {
  readout_ws32<G, FP>(a);
}


// ------------------------------------------------------------ span sums, d = 32, chunk 64
//
// The span sums of the wave-specialised d = 32 readout's plan: 8 waves, wave W
// owning feature tiles W, W + 8, ... (5 or 4 of the 33), key features built by
// lane rotation (as in the readout's state waves), the key Gram matrix on
// wave 7.  The chunk goes from HBM straight into LDS by DMA (raw V rows with
// 16-byte pieces swizzled by vswz(row), raw K rows with pieces swizzled
// by row & 2 against bank conflicts of the transposing reads), three buffers
// deep, each chunk's transfer issued two chunks ahead; the MFMA operands come
// from transposing reads.  The span state is stored in the layout the readout
// loads: value tiles at full scale (key features of weight 2, the products
// here carry 1: stored doubled) and the z column as 2 Z[a][b] on the
// position of each pair.
struct alignas(16) DmaTile32 {
  alignas(16) uint16_t v[64 * DV];  // [token][value column], pieces swizzled by vswz
  alignas(16) uint16_t k[64 * 32];  // [token][dimension], pieces swizzled by row & 2
  alignas(16) float gk[64];         // gated read: key factors 2^((beta_C - beta_t) / 2)
};

// wave W's share of a chunk's transfer: V rows 8 W .. 8 W + 7; waves 4..7
// also K rows 16 (W - 4) .. + 15; gated, wave 0 also the key factors (16
// lanes).  Rows past the end arrive as zero.
template <int W, bool G = false>
__device__ __forceinline__ void dma_chunk32(DmaTile32& b, const ChunkSrc& src, int lane) {
  {
    const int t = 8 * W + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.v[8 * W * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
  if constexpr (W >= 4) {
    const int t = 16 * (W - 4) + (lane >> 2);
    const int c = (lane & 3) ^ (t & 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, KATA_LDS(&b.k[16 * (W - 4) * 32]), 16, t * 64 + 16 * c, 0, 0, 0);
  }
  if constexpr (G && W == 0) {
    if (lane < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(src.gk, KATA_LDS(&b.gk[0]), 16, 16 * lane, 0, 0, 0);
  }
}

// offsets of the transposing K reads: lane (g, s) gets dimension 16 I + s of
// its 8 tokens (rows 4 g + s / 4 of each 16-token half of the k-step)
__device__ __forceinline__ int tr_offset_k32(int I, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = 4 * g + (s >> 2);
  const int c = (2 * I + ((s & 3) >> 1)) ^ ((s >> 2) & 2);
  return row * 32 + 8 * c + 4 * (s & 1);
}

// G: the gated span sums (the state decays by 2^beta_C per chunk, keys scaled
// by the key factors, no Gram matrix; the z column is stored as zeros).
// NH = 2 (fewer spans than CUs): two workgroups per span, each reading the
// whole chunk and reducing every other feature tile of each wave (half h
// takes tiles W + 8 (2 m + h)); blocks b and b + BH (n_spans - 1) hold the
// two halves of a span, on the same XCD when that count is a multiple of 8.
template <bool G, int NH>
__device__ __forceinline__ void span_state_ws32_body(const MfmaArgs& a) {
  using CF = CfgWs32;
  constexpr int C = 64;
  __shared__ DmaTile32 b0;
  __shared__ DmaTile32 b1;
  __shared__ DmaTile32 b2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nsp_work = a.n_spans - 1;  // the last span's sum is never read
  const int64_t nwork = a.BH * nsp_work;
  const int h = static_cast<int>(blockIdx.x / nwork);
  const int64_t blk = blockIdx.x - h * nwork;
  const int64_t bh = blk / nsp_work;
  const int64_t sp = blk - bh * nsp_work;
  const int64_t tok0 = bh * a.T;
  const int64_t first = sp * a.G * C;
  int64_t end = first + a.G * C;
  if (end > a.T) end = a.T;
  auto src = [&](int64_t c) { return chunk_src<32, C>(nullptr, a.k, a.v, tok0, c, end, a.gb, a.gk); };

  auto half = [&](auto hc) {
  with_wave<8>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int H = decltype(hc)::value;
    constexpr int NPC = (W >= 4 ? 2 : 1) + (G && W == 0 ? 1 : 0);  // this wave's transfers per chunk
    constexpr int NFT = mfma_feature_tiles(32);
    constexpr int T0 = W + 8 * H, TS = 8 * NH;  // tiles T0, T0 + TS, ...
    constexpr int MT = (NFT - T0 + TS - 1) / TS;
    constexpr bool GRAM = W == 7 && H == 0 && !G;
    const TrOffsets to = tr_offsets(lane);
    const int ok0 = tr_offset_k32(0, lane), ok1 = tr_offset_k32(1, lane);
    f32x4 acc[MT][NDT - 1];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) acc[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 zt[GRAM ? 4 : 1];
#pragma unroll
    for (int t = 0; t < (GRAM ? 4 : 1); ++t) zt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto reduce = [&](const DmaTile32& b, int64_t c) {
      if constexpr (G) {
        // the state decays by 2^beta_C over the chunk (a whole chunk: beta_C / 2 stored)
        const float f = __builtin_amdgcn_exp2f(2.f * a.gb[tok0 + c + C - 1]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int dt = 0; dt < NDT - 1; ++dt) acc[m][dt] *= f;
        }
      }
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        u32x4 bv[NDT - 1];
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt) bv[dt] = tr_operand<DV>(b.v, to.v[dt], ks);
        const u32x4 k0 = tr_operand<32>(b.k, ok0, ks);
        const u32x4 k1 = tr_operand<32>(b.k, ok1, ks);
        if constexpr (GRAM) {
          zt[0] = mfma(k0, k0, zt[0]);
          zt[1] = mfma(k0, k1, zt[1]);
          zt[2] = mfma(k1, k0, zt[2]);
          zt[3] = mfma(k1, k1, zt[3]);
        }
        float x[2][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[0][2 * i] = lo_bf16(k0[i]);
          x[0][2 * i + 1] = hi_bf16(k0[i]);
          x[1][2 * i] = lo_bf16(k1[i]);
          x[1][2 * i + 1] = hi_bf16(k1[i]);
        }
        if constexpr (G) ws32_gate_keys(x, b.gk, ks, g);
        ws32_key_tiles<T0, TS>(acc, x, bv, r, std::make_integer_sequence<int, MT>{});
      }
    };
    dma_chunk32<W, G>(b0, src(first), lane);
    dma_chunk32<W, G>(b1, src(first + C), lane);
    for (int64_t c0 = first; c0 < end; c0 += 3 * C) {
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk32<W, G>(b2, src(c0 + 2 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      reduce(b0, c0);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk32<W, G>(b0, src(c0 + 3 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (c0 + C < end) reduce(b1, c0 + C);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NPC));
      barrier_lds();
      dma_chunk32<W, G>(b1, src(c0 + 4 * C), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (c0 + 2 * C < end) reduce(b2, c0 + 2 * C);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    // store: value tiles doubled (the state's key features carry weight 2),
    // z as 2 Z[a][b] on the position of each pair a <= b
    float* P = a.ws + (bh * a.n_spans + sp) * mfma_state_floats(32);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int ft = T0 + TS * m;
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) {
        *reinterpret_cast<float4*>(P + ((ft * (NDT - 1) + dt) * 64 + lane) * 4) =
            make_float4(2.f * acc[m][dt][0], 2.f * acc[m][dt][1], 2.f * acc[m][dt][2], 2.f * acc[m][dt][3]);
      }
    }
    if constexpr (GRAM) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int I = t >> 1, J = t & 1;
        if (I > J) continue;  // the mirror of tile (0, 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ra = 16 * I + 4 * g + i, cb = 16 * J + r;
          if (ra <= cb) P[CF::ZOFF + kPairPos32.p[ra][cb]] = 2.f * zt[t][i];
        }
      }
    }
    if constexpr (G && W == 7 && H == 0) {
      // no denominator: the z column holds zeros
      for (int i = lane; i < 16 * NFT; i += 64) P[CF::ZOFF + i] = 0.f;
    }
  });
  };
  if (NH == 1 || h == 0) {
    half(std::integral_constant<int, 0>{});
  } else if constexpr (NH == 2) {
    half(std::integral_constant<int, 1>{});
  }
}

// the d = 32 span sums split over two workgroups per span while the spans do
// not fill the CUs (B=2 H=16 T=8192: span stage 30.0 -> 28.3 us, step 103.2
// -> 101.2 us; B=8 H=16 T=2048 83.3 -> 78.1 us; a fourth and fifth chunk
// buffer instead, or as well, measured slower)
constexpr int64_t kSplitSpanSums32 = 256;

template <bool G = false, int NH = 1>
__global__ __launch_bounds__(512, 2) void span_state_ws32_kernel(MfmaArgs a) {
  span_state_ws32_body<G, NH>(a);
}

// ------------------------------------------------------------ readout, d = 16, LDS DMA
//
// The chunk's V, K and Q arrive raw by LDS DMA into one of two buffers while
// the other is read.  Query rows and score operands are plain row reads; V and
// K operands come from transposing reads, as in the span sums.
template <int C, bool G = false>
struct alignas(16) DmaTileQ16 : GateRows<C, G, false> {
  static constexpr bool kKeyFactors = false;
  alignas(16) uint16_t v[C * DV];  // [token][value column], swizzled
  alignas(16) uint16_t k[C * 16];  // [token][dimension]
  alignas(16) uint16_t q[C * 16];  // [token][dimension]
};

// (WQ false: V and K only, for a chunk whose queries are not read out)
template <int C, int W, int NW, bool G = false, bool WQ = true>
__device__ __forceinline__ void dma_chunkq16(DmaTileQ16<C, G>& b, const ChunkSrc& src, int lane) {
#pragma unroll
  for (int j = W; j < C / 8; j += NW) {
    const int t = 8 * j + (lane >> 3);
    const int cg = (lane & 7) ^ vswz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, KATA_LDS(&b.v[8 * j * DV]), 16, t * (2 * DV) + 16 * cg, 0, 0, 0);
  }
#pragma unroll
  for (int j = W; j < C / 32; j += NW) {
    const int t = 32 * j + (lane >> 1);
    const int pc = (lane & 1) ^ ksw16(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, KATA_LDS(&b.k[32 * j * 16]), 16, t * 32 + 16 * pc, 0, 0, 0);
    if constexpr (WQ)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.q, KATA_LDS(&b.q[32 * j * 16]), 16, t * 32 + 16 * pc, 0, 0, 0);
  }
  dma_gate<G, W, NW>(b, src, lane);
}

template <int C, bool G = false>
struct DmaSrc16 {
  static constexpr bool kGramDen = !G;
  static constexpr bool kHalfDiag = !G;  // Sb's diagonal tile is stored halved
  const DmaTileQ16<C, G>& b;
  const TrOffsets& to;
  const uint16_t* gram;  // bf16 Z, 16 x 16 row-major (ungated read)
  // rows of 32 bytes with their 16-byte pieces swizzled by ksw16(row)
  __device__ __forceinline__ float4 qrow4(int row, int c4) const {
    const uint2 x = *reinterpret_cast<const uint2*>(&b.q[row * 16 + 4 * (c4 ^ (2 * ksw16(row)))]);
    return make_float4(lo_bf16(x.x), hi_bf16(x.x), lo_bf16(x.y), hi_bf16(x.y));
  }
  __device__ __forceinline__ uint2 score_q(int row, int g) const {
    return *reinterpret_cast<const uint2*>(&b.q[row * 16 + 4 * (g ^ (2 * ksw16(row)))]);
  }
  __device__ __forceinline__ uint2 score_k(int row, int g) const {
    return *reinterpret_cast<const uint2*>(&b.k[row * 16 + 4 * (g ^ (2 * ksw16(row)))]);
  }
  __device__ __forceinline__ u32x4 v_op(int vt, int s, int lane) const {
    return tr_operand<DV>(b.v, to.v[vt], s);
  }
  // Z[r][4g .. 4g + 3], the A operand of E = Z Q^T (rows swizzled as K)
  __device__ __forceinline__ uint2 gram_op(int r, int g) const {
    return *reinterpret_cast<const uint2*>(&gram[r * 16 + 4 * (g ^ (2 * ksw16(r)))]);
  }
  __device__ __forceinline__ float gate(int row) const { return b.gb[row]; }
  __device__ __forceinline__ float4 gate4(int row) const {
    return *reinterpret_cast<const float4*>(&b.gb[row]);
  }
};

// state carry of the readout: wave W owns feature tiles W, W + 4 (and 8 for
// wave 0), the whole state being needed for the next chunk's state copy.
// The value tiles only: the ungated read carries z as the Gram matrix
// Z += K^T K (wave 0; the transposing key read is both operands).
template <class CF, int W, bool G = false>
__device__ __forceinline__ void state_update_ro16(f32x4 (&acc)[CF::MFT][NDT], f32x4& gram,
                                                  const DmaTileQ16<CF::C, G>& b, const TrOffsets& to) {
  static_assert((CF::NW == 4 || CF::NW == 8) && CF::NFT == 9, "d = 16 tiling");
  float beta_c = 0.f;
  if constexpr (G) {
    beta_c = b.gb[CF::C - 1];  // beta_C / 2
    gate_decay(acc, __builtin_amdgcn_exp2f(2.f * beta_c));
  }
#pragma unroll
  for (int ks = 0; ks < CF::C / 32; ++ks) {
    u32x4 bv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt) bv[dt] = tr_operand<DV>(b.v, to.v[dt], ks);
    const u32x4 kb = tr_operand<16>(b.k, to.k, ks);
    if constexpr (!G && W == 0) gram = mfma(kb, kb, gram);
    float kr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[2 * i] = kSqrt2 * lo_bf16(kb[i]);
      kr[2 * i + 1] = kSqrt2 * hi_bf16(kb[i]);
    }
    if constexpr (G) gate_keys(kr, b.gb, beta_c, ks);
    constexpr int N = NDT - 1, NW = CF::NW;
    // wave W owns feature tiles W, W + NW, ... (below 9)
    tile16_into<W, N>(acc[0], kr, bv);
    if constexpr (W + NW < 9) tile16_into<W + NW, N>(acc[1], kr, bv);
    if constexpr (W + 2 * NW < 9) tile16_into<W + 2 * NW, N>(acc[2], kr, bv);
  }
}

// d = 16: the key Gram matrix Z = sum_s k_s k_s^T of a span state (zero for
// none).  The state's z column holds, on tile J's row R, 2 Z[R][R + J mod 16]
// (the state's key features carry weight 2 on every pair; see store_gram16);
// Z is symmetric, so each entry sits on a tile J <= 8.  Lane (g, r) gets
// Z[4g + i][r], the accumulator layout.
template <class CF>
__device__ __forceinline__ f32x4 load_gram16(const float* __restrict__ P, int lane) {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  if (P == nullptr) return z;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i, j = (r - row) & 15;
    z[i] = 0.5f * P[CF::ZOFF + (j <= 8 ? 16 * j + row : 16 * (16 - j) + r)];
  }
  return z;
}

// load_gram16 of the sum of the n span sums at P0, P0 + E, ... (summed in
// span order, then halved, as the sequential prefix and load_gram16 do)
template <class CF>
__device__ __forceinline__ f32x4 sum_gram16(const float* __restrict__ P0, int64_t n, int lane) {
  const int g = lane >> 4, r = lane & 15;
  int off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i, j = (r - row) & 15;
    off[i] = CF::ZOFF + (j <= 8 ? 16 * j + row : 16 * (16 - j) + r);
  }
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int64_t s = 0; s < n; ++s) {
    const float* P = P0 + s * mfma_state_floats(CF::DK);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] += P[off[i]];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] *= 0.5f;
  return z;
}

// bf16 copy of Z, row-major with the 16-byte pieces of row r swizzled by
// ksw16(r): lane (g, r) holds Z[4g + i][r] = Z[r][4g + i]
__device__ __forceinline__ void write_gram16(uint16_t* __restrict__ zb, const f32x4& z, int lane) {
  const int g = lane >> 4, r = lane & 15;
  *reinterpret_cast<uint2*>(&zb[16 * r + 4 * (g ^ (2 * ksw16(r)))]) = make_uint2(pack2(z[0], z[1]), pack2(z[2], z[3]));
}

// DMA instructions one readout wave issues per chunk (ungated; WQ: with Q)
template <int C, int W, int NW, bool WQ>
constexpr int dma_count_q16() {
  int n = 0;
  for (int j = W; j < C / 8; j += NW) ++n;
  for (int j = W; j < C / 32; j += NW) n += WQ ? 2 : 1;
  return n;
}

// a tile that exists only when E holds (an empty struct otherwise)
template <bool E, class T>
struct MaybeTile {
  T t;
};
template <class T>
struct MaybeTile<false, T> {};

// Span of a workgroup that forms its prefix itself (RC): the latest spans,
// which carry the most chunks before them, take the lowest block indices and
// start first; consecutive blocks are different heads.
__device__ inline SpanOf recompute_span(const MfmaArgs& a) {
  const int64_t b = blockIdx.x;
  return {b % a.BH, a.n_spans - 1 - b / a.BH};
}

// The kernel body, a device function taking the arguments by reference (this
// form compiles to slightly fewer registers and branches than the body in the
// kernel itself, and measured 2% faster at T = 131072).
//
// Denominators (ungated read): no ones-column tile.  Wave 0 carries the key
// Gram matrix Z (one 16x16x32 product per 32 keys, against 9 for a ones
// column over the feature tiles) and publishes its bf16 copy with Sb.
//
// RC (prefix formed in the workgroup, for heads of few spans): no prefix
// state is read.  The workgroup starts at the head's first chunk and carries
// the state from zero over every chunk before its span (keys and values
// only, nothing read out), then reads out its span as usual.  The exclusive
// prefix of Eqs. 17-20 is then summed chunk by chunk in one workgroup, with
// no span-sum or prefix launch; every span of a head repeats that sum.
// FP (a.fused): the span sums of the spans before this one are stored
// unscanned; the workgroup adds them in span order in its prologue.
template <int C, bool G, bool RC = false, bool FP = false>
__device__ __forceinline__ void readout_dma16_body(const MfmaArgs& a) {
  using CF = Cfg<16, C>;
  constexpr int DK = 16, SB_LD = CF::SB_LD;
  static_assert(CF::NDW == NDT, "whole output rows per wave");
  static_assert(!(G && RC) && !(G && FP) && !(RC && FP), "one prefix source per readout");
  __shared__ DmaTileQ16<C, G> x0;
  __shared__ DmaTileQ16<C, G> x1;
  // the third buffer of the deep warm-up (prefix formed in the workgroup, chunk 64)
  constexpr bool DEEP = RC && C == 64;
  __shared__ MaybeTile<DEEP, DmaTileQ16<C, G>> x2h;
  // bf16 Z (the gated read has no denominator)
  __shared__ alignas(16) uint16_t Zb[G ? 4 : 256];
  // value rows only: this readout keeps no z column in Sb
  __shared__ alignas(16) uint16_t Sb[DV * SB_LD];
  __shared__ alignas(16) uint16_t Ob[CF::STAGE_OUT ? CF::NW : 1][16 * OB_LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SpanOf span = RC ? recompute_span(a) : FP ? fused_span(a) : readout_span(a);
  const int64_t bh = span.bh, sp = span.sp;
  const int64_t tok0 = bh * a.T;

  with_wave<CF::NW>(w, [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    // output stores a wave issues per chunk: two 1 KB stores per query tile,
    // or one 8-byte store per value tile without the LDS staging
    constexpr int NSTORE = (CF::STAGE_OUT ? 2 : NDT - 1) * CF::NSLOT;
    const ReadoutLane<CF> L = readout_lane<CF>(W, lane);
    const TrOffsets to = tr_offsets(lane);
    const int64_t first = span_first_chunk(a, sp) * C;
    int64_t end = span_first_chunk(a, sp + 1) * C;
    if (end > a.T) end = a.T;
    auto src = [&](int64_t c) { return chunk_src<DK, C>(a.q, a.k, a.v, tok0, c, end, a.gb, a.gk); };
    const int64_t start = (RC && !DEEP) ? 0 : first;
    // the first chunk's transfer goes out before the prefix state is read,
    // so the two HBM latencies overlap (the warm-up of DEEP issues its own)
    if constexpr (!DEEP) dma_chunkq16<C, W, CF::NW, G>(x0, src(start), lane);
    f32x4 acc[CF::MFT][NDT];
    const float* prefix =
        (!RC && !FP && a.n_spans > 1) ? a.ws + (bh * a.n_spans + sp) * mfma_state_floats(DK) : nullptr;
    const float* sums = FP ? a.ws + bh * a.n_spans * mfma_state_floats(DK) : nullptr;
    if constexpr (FP) {
      sum_states<CF>(acc, sums, sp, W, lane);
    } else {
      load_state<CF>(acc, prefix, W, lane);
    }
    // feature positions no tile writes hold no feature: zero once (the 16
    // positions of tile 8 in lane groups 2 and 3, below)
    for (int e = tid; e < DV * 16; e += CF::NT) {
      const int j = e & 15;
      Sb[(e >> 4) * SB_LD + 128 + 8 * (j >> 2) + 4 + (j & 3)] = 0;
    }
    // the d = 16 span sums store the value tiles at kSpanValueScale
#pragma unroll
    for (int m = 0; m < CF::MFT; ++m) {
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) acc[m][dt] *= 1.f / kSpanValueScale;
    }
    write_sb<CF, NDT - 1, DmaSrc16<C, G>::kHalfDiag>(Sb, acc, W, lane);
    f32x4 gram = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!G && W == 0) {
      gram = FP ? sum_gram16<CF>(sums, sp, lane) : load_gram16<CF>(prefix, lane);
      write_gram16(Zb, gram, lane);
    }
    bool staged = !DEEP;  // chunk `start` already on its way into x0
    if constexpr (DEEP) {
      // The chunks before the span, three buffers deep: step i waits for its
      // own share of chunk i, meets the other waves at a barrier (after which
      // nobody reads chunk i - 1's buffer), sends chunk i + 2 into that
      // buffer (queries only for the span's first chunk) and adds chunk i to
      // the state.  Chunk i sits in buffer (i - nf) mod 3 of (x0, x1, x2), so
      // the span's first chunk (index nf) arrives in x0.  Steps before chunk 0
      // only issue the first two transfers.
      const int64_t nf = first / C;
      if (nf > 0) {
        constexpr int NK = dma_count_q16<C, W, CF::NW, false>();
        constexpr int NQ = dma_count_q16<C, W, CF::NW, true>();
        auto wstep = [&](int64_t i, const DmaTileQ16<C, G>& cur, DmaTileQ16<C, G>& pre) {
          if (i >= 0 && i < nf) {
            if (i + 1 == nf) {
              __builtin_amdgcn_s_waitcnt(wait_vmcnt(NQ));
            } else {
              __builtin_amdgcn_s_waitcnt(wait_vmcnt(NK));
            }
            barrier_lds();
          }
          if (i + 2 >= 0 && i + 2 <= nf) {
            __builtin_amdgcn_sched_barrier(0);
            if (i + 2 == nf) {
              dma_chunkq16<C, W, CF::NW, G>(pre, src((i + 2) * C), lane);
            } else {
              dma_chunkq16<C, W, CF::NW, G, false>(pre, src((i + 2) * C), lane);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if (i >= 0 && i < nf) state_update_ro16<CF, W, G>(acc, gram, cur, to);
        };
        const int64_t s0 = nf - 3 * ((nf + 2) / 3 + 1);  // <= -3, s0 = nf (mod 3)
        for (int64_t i = s0; i < nf; i += 3) {
          wstep(i, x0, x2h.t);
          wstep(i + 1, x1, x0);
          wstep(i + 2, x2h.t, x1);
        }
        // the span's first chunk has landed (the last transfer issued)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        write_sb<CF, NDT - 1, DmaSrc16<C, G>::kHalfDiag>(Sb, acc, W, lane);
        if constexpr (!G && W == 0) write_gram16(Zb, gram, lane);
        __syncthreads();
        staged = true;
      }
    }
    if (!DEEP || !staged) {
      if (!staged) dma_chunkq16<C, W, CF::NW, G>(x0, src(start), lane);
      // the state loads and the first chunk; an unconditional vmcnt(0) also
      // retires the state loads for the compiler's wait-count analysis
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }

    // one chunk: prefetch the next into the other buffer, read out, and
    // (unless it is the span's last) carry the state and refresh Sb
    auto chunk = [&](DmaTileQ16<C, G>& cur, DmaTileQ16<C, G>& nxt, int64_t c) {
      if constexpr (RC) {
        if (c < first) {
          // a chunk before the span: fetch the next (its queries only if it
          // is read out), carry the state, and publish it before the span
          __builtin_amdgcn_sched_barrier(0);
          if (c + C < first) {
            dma_chunkq16<C, W, CF::NW, G, false>(nxt, src(c + C), lane);
          } else {
            dma_chunkq16<C, W, CF::NW, G>(nxt, src(c + C), lane);
          }
          __builtin_amdgcn_sched_barrier(0);
          state_update_ro16<CF, W, G>(acc, gram, cur, to);
          __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
          barrier_lds();
          if (c + C == first) {
            write_sb<CF, NDT - 1, DmaSrc16<C, G>::kHalfDiag>(Sb, acc, W, lane);
            if constexpr (!G && W == 0) write_gram16(Zb, gram, lane);
            barrier_lds();
          }
          return;
        }
      }
      const int64_t n = (a.T - c < C) ? a.T - c : C;
      // the next chunk's transfer goes out right after the query rows are
      // read (zeros past the span's end); issued any earlier, the compiler's
      // wait counts make those row reads wait for it
      auto prefetch = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        dma_chunkq16<C, W, CF::NW, G>(nxt, src(c + C), lane);
        __builtin_amdgcn_sched_barrier(0);
      };
      readout_chunk<CF, DmaSrc16<C, G>, decltype(prefetch), G>(
          DmaSrc16<C, G>{cur, to, Zb}, Sb, L, lane, a.eps, rows_rsrc(a.out, tok0 + c, n, 2 * DV),
          Ob[CF::STAGE_OUT ? W : 0],
          prefetch);
      const bool more = c + C < end;
      if (more) state_update_ro16<CF, W, G>(acc, gram, cur, to);
      // this wave's share of the next chunk has landed (the output stores
      // issued after it may still be in flight).  Unconditional, so that on
      // every path the compiler's wait counts see the transfer retired.
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NSTORE));
      if (more) {
        // every wave is done reading `cur` and Sb, and the next chunk is visible
        barrier_lds();
        write_sb<CF, NDT - 1, DmaSrc16<C, G>::kHalfDiag>(Sb, acc, W, lane);
        if constexpr (!G && W == 0) write_gram16(Zb, gram, lane);
        barrier_lds();
      }
    };
    for (int64_t c0 = start; c0 < end; c0 += 2 * C) {
      chunk(x0, x1, c0);
      if (c0 + C < end) chunk(x1, x0, c0 + C);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  });
}

template <int C, bool G = false, bool RC = false, bool FP = false>
__global__ __launch_bounds__(256, 2) void readout_dma16_kernel(MfmaArgs a) {
  readout_dma16_body<C, G, RC, FP>(a);
}

template <int DK, int C>
hipError_t launch_span(const MfmaArgs& a, hipStream_t stream) {
  using CF = Cfg<DK, C>;
  dim3 grid(static_cast<unsigned>(a.BH * (a.n_spans - 1)));
  if constexpr (DK == 16) {
    // four chunk buffers: 43 KB at chunk 64; at chunk 128 (86 KB, one
    // workgroup per CU) the short form measured slower (B=4 H=8 T=2048 step
    // 21.5 -> 22.1 us; chunk 64: 23.1 -> 22.5 us, B=4 H=8 T=4096 31.7 -> 30.9)
    if (C == 64 && a.GL == 0 && a.G <= 4) {
      span_state_dma16_kernel<C, false, C == 64><<<grid, CF::NT, 0, stream>>>(a);
    } else {
      span_state_dma16_kernel<C><<<grid, CF::NT, 0, stream>>>(a);
    }
  } else if (DK >= 64 && grid.x <= kSplitSpanSums32) {
    // the d = 64 maps: two workgroups per span while the spans do not fill
    // the CUs (B=8 H=16, T=4096: KATA-M4 step 0.265 -> 0.252 ms, M1 1.068
    // -> 1.015 ms; T=131072: M4 7.68 -> 7.20 ms, M1 31.3 -> 29.0 ms); at
    // d = 32, chunk 128 it measured slower (B=2 H=16 T=8192 116.8 -> 122.7 us)
    span_state_mfma_kernel<CF, false, 2><<<dim3(2 * grid.x), CF::NT, 0, stream>>>(a);
  } else {
    span_state_mfma_kernel<CF><<<grid, CF::NT, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int DK, int C>
hipError_t launch_readout(const MfmaArgs& a, hipStream_t stream) {
  using CF = Cfg<DK, C>;
  dim3 grid(static_cast<unsigned>(a.BH * a.n_spans));
  if constexpr (DK == 16) {
    if (a.recompute) {
      readout_dma16_kernel<C, false, true><<<grid, CF::NT, 0, stream>>>(a);
    } else if (a.fused) {
      readout_dma16_kernel<C, false, false, true><<<grid, CF::NT, 0, stream>>>(a);
    } else {
      readout_dma16_kernel<C><<<grid, CF::NT, 0, stream>>>(a);
    }
  } else {
    readout_mfma_kernel<CF><<<grid, CF::NT, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_span_state_mfma(const MfmaArgs& a, hipStream_t stream) {
  if (a.n_spans < 2) return hipSuccess;
  if (a.fm >= 100 && a.chunk == 64) {
    switch (a.fm) {
      case 100: return launch_span<100, 64>(a, stream);
      case 101: return launch_span<101, 64>(a, stream);
      case 102: return launch_span<102, 64>(a, stream);
      case 103: return launch_span<103, 64>(a, stream);
      case 200: return launch_span<200, 64>(a, stream);
      case 201: return launch_span<201, 64>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.d == 16 && a.chunk == 64) return launch_span<16, 64>(a, stream);
  if (a.d == 16 && a.chunk == 128) return launch_span<16, 128>(a, stream);
  if (a.d == 32 && a.chunk == 64) {
    const int64_t spans = a.BH * (a.n_spans - 1);
    if (spans <= kSplitSpanSums32) {
      span_state_ws32_kernel<false, 2><<<dim3(static_cast<unsigned>(2 * spans)), 512, 0, stream>>>(a);
    } else {
      span_state_ws32_kernel<false><<<dim3(static_cast<unsigned>(spans)), 512, 0, stream>>>(a);
    }
    return hipGetLastError();
  }
  if (a.d == 32 && a.chunk == 128) return launch_span<32, 128>(a, stream);
  if (a.d == 64 && a.chunk == 64) return launch_span<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_span_state_gated(const MfmaArgs& a, hipStream_t stream) {
  if (a.n_spans < 2) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.BH * (a.n_spans - 1)));
  if (a.d == 16 && a.chunk == 64) {
    span_state_dma16_kernel<64, true><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 16 && a.chunk == 128) {
    span_state_dma16_kernel<128, true><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 32 && a.chunk == 64) {
    span_state_ws32_kernel<true><<<grid, 512, 0, stream>>>(a);
  } else if (a.d == 32 && a.chunk == 128) {
    span_state_mfma_kernel<Cfg<32, 128>, true><<<grid, Cfg<32, 128>::NT, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_readout_gated(const MfmaArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.BH * a.n_spans));
  if (a.d == 16 && a.chunk == 64) {
    readout_dma16_kernel<64, true><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 16 && a.chunk == 128) {
    readout_dma16_kernel<128, true><<<grid, 256, 0, stream>>>(a);
  } else if (a.d == 32 && a.chunk == 64) {
    readout_ws32_kernel<true><<<grid, 512, 0, stream>>>(a);
  } else if (a.d == 32 && a.chunk == 128) {
    readout_mfma_kernel<Cfg<32, 128>, true><<<grid, Cfg<32, 128>::NT, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_readout_mfma(const MfmaArgs& a, hipStream_t stream) {
  if (a.fm >= 100 && a.chunk == 64) {
    switch (a.fm) {
      case 100: return launch_readout<100, 64>(a, stream);
      case 101: return launch_readout<101, 64>(a, stream);
      case 102: return launch_readout<102, 64>(a, stream);
      case 103: return launch_readout<103, 64>(a, stream);
      case 200: return launch_readout<200, 64>(a, stream);
      case 201: return launch_readout<201, 64>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.d == 16 && a.chunk == 64) return launch_readout<16, 64>(a, stream);
  if (a.d == 16 && a.chunk == 128) return launch_readout<16, 128>(a, stream);
  if (a.d == 32 && a.chunk == 64) {
    if (a.fused) {
      readout_ws32_kernel<false, true><<<dim3(static_cast<unsigned>(a.BH * a.n_spans)), 512, 0, stream>>>(a);
    } else {
      readout_ws32_kernel<false><<<dim3(static_cast<unsigned>(a.BH * a.n_spans)), 512, 0, stream>>>(a);
    }
    return hipGetLastError();
  }
  if (a.d == 32 && a.chunk == 128) return launch_readout<32, 128>(a, stream);
  if (a.d == 64 && a.chunk == 64) return launch_readout<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace kata
