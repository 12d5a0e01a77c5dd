// Tiered gather-GEMV (gfx950), with an optional fused tier selection.
//
// SpAx page, section 2 Eq. 1 and section 5, Figure 2 steps 3-5:
//   y = sum_{j in F} x_j W~[:, j] + sum_{j in A} x_j W^[:, j]
// where W~ is the stored full tier (fp16, or int4 group-128 dequantised) and
// W^ the middle tier rebuilt from int4 / int2 group-128 codes in registers.
// Skipped columns are never touched. This is a matrix-vector product, so it
// runs on the vector ALUs and is bound by HBM bandwidth, not on MFMA.
//
// Work decomposition
//   * Rows are cut into tiles of 512 (64 lanes x 8 rows). Lane l of every
//     wave owns rows row0 + 8l .. row0 + 8l + 7 for all three formats, so the
//     tiers accumulate into the same 8 fp32 registers:
//       fp16 column segment: 1 KB, one 16-byte load per lane;
//       int4 column segment: 256 B, one 4-byte load per lane;
//       int2 column segment: 128 B, one 2-byte load per lane.
//     Every wave-wide load reads one column's contiguous segment.
//   * The selected columns form one virtual list [F..., A...]; it is cut into
//     n_splits pieces of equal bytes. Workgroup (split, tile) streams its
//     piece for its tile; its 8 waves take contiguous eighths of the piece.
//   * Where the list comes from:
//       kListGlobal  index lists in device memory (spax_tiered_gemv); column
//                    indices and activations are fetched 64 at a time (one
//                    per lane) and broadcast with readlane;
//       kListStaged  the selected columns were copied to staging in list
//                    order (host-resident weights);
//       kListRank    the workgroup ranks x itself (tier selection of section
//                    5, Figure 2 step 3) and keeps its own piece of the list,
//                    with the activations, in LDS. Every workgroup reaches the
//                    same boundaries, so no list crosses global memory before
//                    the product; the tile-0 workgroups also write the lists
//                    out for the caller.
//   * Code tiers fold x_j * s_{j,g} into one fp32 factor per column and lane
//     and accumulate the unsigned code; the code offset (8 for int4, 1.5 for
//     int2) is removed once at the end through a per-lane running sum.
//   * The 8 wave partials are added in LDS in a fixed order. With one split
//     the workgroup writes y; otherwise each workgroup stores its fp32 partial
//     and the last workgroup of a tile (agent-scope counter) adds the n_splits
//     partials in split order and writes y. The counter is reset by that
//     workgroup. The summation order never depends on timing, so results are
//     bitwise reproducible.
//   * The tiles of one split run on one XCD (blocks are dealt to the 8 XCDs
//     round-robin), so the shared lines of a split hit that XCD's L2.
//   * Gate/up epilogue: with the GLU-interleaved layout a tile holds 256 gate
//     rows and the matching 256 up rows, so the final reduction forms
//     a = silu(g) * u (SpAx page, section 2) from the fp16-rounded g and u.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "spax_internal.h"

namespace spax {
namespace {

__device__ __forceinline__ float h2f(uint32_t bits) {
  return __half2float(__ushort_as_half((unsigned short)bits));
}
__device__ __forceinline__ uint16_t f2h(float v) {
  return __half_as_ushort(__float2half_rn(v));
}
__device__ __forceinline__ float b2f(uint32_t v, int byte) {
  return (float)((v >> (8 * byte)) & 0xFFu);
}

template <int FMT>
struct Tier;

template <>
struct Tier<kFp16> {
  using V = uint4;
  static constexpr int U = 8;
  static __device__ __forceinline__ V load(const uint8_t* col, int row0, int lane) {
    return *reinterpret_cast<const uint4*>(col + 2 * (size_t)(row0 + 8 * lane));
  }
  static __device__ __forceinline__ void fma(float (&acc)[8], float&, V v, float xs, float) {
    acc[0] = fmaf(h2f(v.x & 0xFFFFu), xs, acc[0]);
    acc[1] = fmaf(h2f(v.x >> 16), xs, acc[1]);
    acc[2] = fmaf(h2f(v.y & 0xFFFFu), xs, acc[2]);
    acc[3] = fmaf(h2f(v.y >> 16), xs, acc[3]);
    acc[4] = fmaf(h2f(v.z & 0xFFFFu), xs, acc[4]);
    acc[5] = fmaf(h2f(v.z >> 16), xs, acc[5]);
    acc[6] = fmaf(h2f(v.w & 0xFFFFu), xs, acc[6]);
    acc[7] = fmaf(h2f(v.w >> 16), xs, acc[7]);
  }
};

template <>
struct Tier<kInt4> {
  using V = uint32_t;
  static constexpr int U = 16;
  static __device__ __forceinline__ V load(const uint8_t* col, int row0, int lane) {
    return *reinterpret_cast<const uint32_t*>(col + (size_t)(row0 + 8 * lane) / 2);
  }
  // Rows 2b and 2b+1 sit in the low and high nibble of byte b, as
  // two's-complement q; flipping each nibble's sign bit gives u = q + 8.
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float xs,
                                             float scale) {
    const float c = xs * scale;  // exact: product of two fp16 values
    corr = fmaf(8.0f, c, corr);
    v ^= 0x88888888u;
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    acc[0] = fmaf(c, b2f(lo, 0), acc[0]);
    acc[1] = fmaf(c, b2f(hi, 0), acc[1]);
    acc[2] = fmaf(c, b2f(lo, 1), acc[2]);
    acc[3] = fmaf(c, b2f(hi, 1), acc[3]);
    acc[4] = fmaf(c, b2f(lo, 2), acc[4]);
    acc[5] = fmaf(c, b2f(hi, 2), acc[5]);
    acc[6] = fmaf(c, b2f(lo, 3), acc[6]);
    acc[7] = fmaf(c, b2f(hi, 3), acc[7]);
  }
};

template <>
struct Tier<kInt2> {
  using V = uint32_t;
  static constexpr int U = 16;
  static __device__ __forceinline__ V load(const uint8_t* col, int row0, int lane) {
    return *reinterpret_cast<const uint16_t*>(col + (size_t)(row0 + 8 * lane) / 4);
  }
  // Row 4b + r sits in bits 2r..2r+1 of byte b; masking leaves u * 4^r, so
  // the factor is scaled by 4^-r (exact).
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float xs,
                                             float scale) {
    const float c = xs * scale;
    corr = fmaf(1.5f, c, corr);
    const uint32_t m0 = v & 0x0303u, m1 = v & 0x0C0Cu, m2 = v & 0x3030u, m3 = v & 0xC0C0u;
    const float c1 = c * 0.25f, c2 = c * 0.0625f, c3 = c * 0.015625f;
    acc[0] = fmaf(c, b2f(m0, 0), acc[0]);
    acc[4] = fmaf(c, b2f(m0, 1), acc[4]);
    acc[1] = fmaf(c1, b2f(m1, 0), acc[1]);
    acc[5] = fmaf(c1, b2f(m1, 1), acc[5]);
    acc[2] = fmaf(c2, b2f(m2, 0), acc[2]);
    acc[6] = fmaf(c2, b2f(m2, 1), acc[6]);
    acc[3] = fmaf(c3, b2f(m3, 0), acc[3]);
    acc[7] = fmaf(c3, b2f(m3, 1), acc[7]);
  }
};

// Per-lane metadata of one 64-column batch of a tier: lane l holds the
// column index and activation of batch position l and, for code tiers, the
// tile's four group scales of that column (groups 0,1 in sc01, 2,3 in sc23).
struct Meta {
  int idx;
  uint32_t xb;  // fp16 bits (global modes) or fp32 bits (rank mode)
  uint32_t sc01, sc23;
};

template <int FMT, int MODE>
__device__ __forceinline__ Meta load_meta(const uint16_t* __restrict__ scales, int64_t sstride,
                                          const int32_t* __restrict__ idx,
                                          const uint16_t* __restrict__ x, const int32_t* lidx,
                                          const float* lx, int p, int cnt, int row0, int ngrp,
                                          int lane) {
  Meta m{0, 0u, 0u, 0u};
  if (cnt <= 0) return m;
  // lanes past the batch repeat its first position (in range, never used)
  const int q = p + (lane < cnt ? lane : 0);
  if constexpr (MODE == kListRank) {
    m.idx = lidx[q];
    m.xb = __float_as_uint(lx[q]);
  } else {
    m.idx = idx[q];
    m.xb = x[m.idx];
  }
  if constexpr (FMT == kInt4 || FMT == kInt2) {
    const int64_t col = MODE == kListStaged ? (int64_t)q : (int64_t)m.idx;
    const uint16_t* sp = scales + col * sstride + (row0 >> 7);
    const uint32_t g0 = sp[0];
    const uint32_t g1 = ngrp > 1 ? sp[1] : 0u;
    const uint32_t g2 = ngrp > 2 ? sp[2] : 0u;
    const uint32_t g3 = ngrp > 3 ? sp[3] : 0u;
    m.sc01 = g0 | (g1 << 16);
    m.sc23 = g2 | (g3 << 16);
  }
  return m;
}

template <int MODE>
__device__ __forceinline__ float meta_x(const Meta& m, int c) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)m.xb, c);
  if constexpr (MODE == kListRank) return __uint_as_float(b);
  else return h2f(b);
}

// This lane's group scale of batch column c (hi_pair: groups 2,3; sh: 0 or 16).
__device__ __forceinline__ float meta_scale(const Meta& m, int c, bool hi_pair, uint32_t sh) {
  const uint32_t a01 = (uint32_t)__builtin_amdgcn_readlane((int)m.sc01, c);
  const uint32_t a23 = (uint32_t)__builtin_amdgcn_readlane((int)m.sc23, c);
  return h2f(((hi_pair ? a23 : a01) >> sh) & 0xFFFFu);
}

template <int MODE>
__device__ __forceinline__ int meta_col(const Meta& m, int p, int c) {
  return MODE == kListStaged ? p + c : __builtin_amdgcn_readlane(m.idx, c);
}

// Multiply-add U loaded columns of one tier; slots u >= n were loaded from
// a valid column and are added with a zero activation.
template <typename T, int MODE>
__device__ __forceinline__ void consume(float (&acc)[8], float& corr,
                                        const typename T::V (&v)[T::U], const Meta& m, int c0,
                                        int n, bool hi_pair, uint32_t sh, bool code) {
#pragma unroll
  for (int u = 0; u < T::U; ++u) {
    const int c = c0 + (u < n ? u : 0);
    const float xs = u < n ? meta_x<MODE>(m, c) : 0.0f;
    const float sc = code ? meta_scale(m, c, hi_pair, sh) : 0.0f;
    T::fma(acc, corr, v[u], xs, sc);
  }
}

// Stream this wave's full-tier list positions [f_lo, f_hi) and approx-tier
// positions [a_lo, a_hi) for its rows. Each round issues the loads of up to
// UF full columns and UA code columns before any of them is consumed, so a
// wave keeps both tiers' bytes in flight together; the last, partial round
// of a batch issues only the loads it needs (wave-uniform guards).
//   kListGlobal: idx lists and x in device memory;
//   kListStaged: columns staged in list order (column = position);
//   kListRank:   lidx / lx = this workgroup's list piece in LDS.
template <int FF, int AF, int MODE>
__device__ __forceinline__ void stream_tiers(float (&acc)[8], float& corr, const GemvArgs& a,
                                             const int32_t* lidx, const float* lx, int f_lo,
                                             int f_hi, int a_lo, int a_hi, int row0, int lane,
                                             int ld_lane) {
  using TF = Tier<FF>;
  using TA = Tier<AF == kNone ? kInt4 : AF>;
  constexpr int UF = TF::U;
  constexpr int UA = AF == kNone ? 0 : TA::U;
  const int grp = ld_lane >> 4;  // this lane's group in the tile
  const bool hi_pair = grp >= 2;
  const uint32_t sh = 16u * (uint32_t)(grp & 1);
  const int ngrp = min(4, (a.rows - row0 + kGroup - 1) / kGroup);
  if constexpr (AF == kNone) a_hi = a_lo;
  // rank mode: the approx part of the piece follows the full part in LDS
  int pf = f_lo, pa = a_lo;
  while (pf < f_hi || pa < a_hi) {
    const int nbf = min(64, f_hi - pf), nba = min(64, a_hi - pa);
    const Meta mf = load_meta<FF, MODE>(a.full_scales, a.full_sstride, a.full_idx, a.x, lidx, lx,
                                        pf, nbf, row0, ngrp, lane);
    Meta ma{0, 0u, 0u, 0u};
    if constexpr (AF != kNone)
      ma = load_meta<AF, MODE>(a.approx_scales, a.approx_sstride, a.approx_idx, a.x, lidx, lx,
                               pa, nba, row0, ngrp, lane);
    for (int cf = 0, ca = 0; cf < nbf || ca < nba; cf += UF, ca += UA) {
      // Slots past the batch reload the round's first column and add it
      // times zero, so every load of a round is issued unconditionally.
      const int nf = min(UF, nbf - cf), na = min(UA, nba - ca);
      if (nf > 0) {
        typename TF::V vf[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
          const int c = cf + (u < nf ? u : 0);
          vf[u] = TF::load(a.full_base + (int64_t)meta_col<MODE>(mf, pf, c) * a.full_stride, row0,
                           ld_lane);
        }
        if constexpr (AF != kNone) {
          if (na > 0) {
            typename TA::V va[UA > 0 ? UA : 1];
#pragma unroll
            for (int u = 0; u < UA; ++u) {
              const int c = ca + (u < na ? u : 0);
              va[u] = TA::load(
                  a.approx_base + (int64_t)meta_col<MODE>(ma, pa, c) * a.approx_stride, row0,
                  ld_lane);
            }
            consume<TF, MODE>(acc, corr, vf, mf, cf, nf, hi_pair, sh, FF != kFp16);
            consume<TA, MODE>(acc, corr, va, ma, ca, na, hi_pair, sh, true);
            continue;
          }
        }
        consume<TF, MODE>(acc, corr, vf, mf, cf, nf, hi_pair, sh, FF != kFp16);
      } else if constexpr (AF != kNone) {
        typename TA::V va[UA > 0 ? UA : 1];
#pragma unroll
        for (int u = 0; u < UA; ++u) {
          const int c = ca + (u < na ? u : 0);
          va[u] = TA::load(a.approx_base + (int64_t)meta_col<MODE>(ma, pa, c) * a.approx_stride,
                           row0, ld_lane);
        }
        consume<TA, MODE>(acc, corr, va, ma, ca, na, hi_pair, sh, true);
      }
    }
    pf += max(nbf, 0);
    pa += max(nba, 0);
  }
}

// Block -> (split, tile): groups of 8 consecutive splits are interleaved so
// that block b and split (b mod 8) coincide on the XCD that runs block b.
__device__ __forceinline__ void map_block(int b, int n_tiles, int splits_here, int& s_loc,
                                          int& tile) {
  const int groups = splits_here >> 3;
  const int fb = groups * 8 * n_tiles;
  if (b < fb) {
    const int g = b / (8 * n_tiles);
    const int r = b - g * 8 * n_tiles;
    s_loc = g * 8 + (r & 7);
    tile = r >> 3;
  } else {
    const int r = b - fb;
    s_loc = groups * 8 + r / n_tiles;
    tile = r % n_tiles;
  }
}

// ---------------------------------------------------------------------------
// In-workgroup tier selection (kListRank). Same definition as the stand-alone
// plan kernel: order key = fp16 magnitude bits, larger first, lower index
// first among equal keys; the k_full first are F, the next k_approx are A.
// Thread t owns entries [t*E, t*E+E).
//   1. 256-bin histogram of key bits 14..7 (per-wave LDS histograms);
//   2. suffix counts give the bins holding rank k_full and k_full + k_approx;
//   3. 128-bin histograms inside those bins give the boundary keys t1, t2
//      and the number of entries equal to each that are kept (q1, q2);
//   4. one block scan of (#key > t1, #key == t1, #key > t2, #key == t2) gives
//      every entry its position: #F before entry i is
//      gt1(i) + min(eq1(i), q1), #(F or A) before it gt2(i) + min(eq2(i), q2).
// ---------------------------------------------------------------------------
constexpr uint32_t kAboveAll = 0x8000u;  // boundary key when a tier is empty

struct RankShared {
  uint32_t hist[kWaves][256];
  uint32_t sub[2][128];
  uint32_t scan[4][kWaves];
  int32_t sel[8];
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (lanes whose source is outside the row add 0).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Sum of v over the lanes above this one.
__device__ __forceinline__ uint32_t wave_excl_suffix(uint32_t v) {
  const uint32_t incl = wave_incl_scan(v);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  return total - incl;
}

__device__ __forceinline__ uint32_t rawbits(const uint32_t* xr, int i) {
  return (xr[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

// Ranks x and places this workgroup's list positions in LDS: full-tier
// positions [f0, f1) at slots [0, f1 - f0), approx-tier positions [a0, a1)
// after them.
template <int E>
__device__ __forceinline__ void rank_piece(const GemvArgs& a, RankShared& rs, int32_t* lidx,
                                           float* lx, int f0, int f1, int a0, int a1,
                                           bool write_lists) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int n = a.n;
  const int base = t * E;
  const uint32_t K1 = (uint32_t)a.k_full;
  const uint32_t K2 = (uint32_t)(a.k_full + a.k_approx);

  // raw fp16 bits, two per register
  uint32_t xr[E / 2];
#pragma unroll
  for (int i = 0; i < E; i += 8) {
    if (base + i + 7 < n) {
      const uint4 v = *reinterpret_cast<const uint4*>(a.x + base + i);
      xr[i / 2 + 0] = v.x;
      xr[i / 2 + 1] = v.y;
      xr[i / 2 + 2] = v.z;
      xr[i / 2 + 3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t lo = base + i + j < n ? a.x[base + i + j] : 0u;
        const uint32_t hi = base + i + j + 1 < n ? a.x[base + i + j + 1] : 0u;
        xr[(i + j) / 2] = lo | (hi << 16);
      }
    }
  }
  const int nv = max(0, min(E, n - base));  // valid entries of this thread

  for (int i = t; i < kWaves * 256; i += kGemvThreads) (&rs.hist[0][0])[i] = 0u;
  if (t < 256) (&rs.sub[0][0])[t] = 0u;
  if (t == 0) {
    rs.sel[0] = -1; rs.sel[1] = 0; rs.sel[2] = -1; rs.sel[3] = 0;
    rs.sel[4] = (int32_t)kAboveAll; rs.sel[5] = 0; rs.sel[6] = (int32_t)kAboveAll; rs.sel[7] = 0;
  }
  __syncthreads();

  // 1. top-level histogram
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (i < nv) atomicAdd(&rs.hist[wave][(rawbits(xr, i) & 0x7FFFu) >> 7], 1u);
  __syncthreads();
  if (t < 256) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += rs.hist[w][t];
    rs.hist[0][t] = s;  // only this thread reads column t
  }
  __syncthreads();

  // 2. bins holding rank K1 and rank K2 (1-based, from the largest key)
  if (wave == 0) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = rs.hist[0][4 * lane + j];
    uint32_t above = wave_excl_suffix(c[0] + c[1] + c[2] + c[3]);
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (K1 > 0 && above < K1 && K1 <= above + c[j]) {
        rs.sel[0] = 4 * lane + j;
        rs.sel[1] = (int32_t)above;
      }
      if (K2 > 0 && above < K2 && K2 <= above + c[j]) {
        rs.sel[2] = 4 * lane + j;
        rs.sel[3] = (int32_t)above;
      }
      above += c[j];
    }
  }
  __syncthreads();

  // 3. low-level histograms inside the two boundary bins
  const int b1 = rs.sel[0];
  const int b2 = rs.sel[2];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i >= nv) continue;
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const int hb = (int)(k >> 7);
    if (hb == b1) atomicAdd(&rs.sub[0][k & 127u], 1u);
    if (hb == b2) atomicAdd(&rs.sub[1][k & 127u], 1u);
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = r == 0 ? b1 : b2;
      const uint32_t K = r == 0 ? K1 : K2;
      if (b < 0) continue;
      const uint32_t c0 = rs.sub[r][2 * lane], c1 = rs.sub[r][2 * lane + 1];
      uint32_t above = (uint32_t)rs.sel[1 + 2 * r] + wave_excl_suffix(c0 + c1);
      if (above < K && K <= above + c1) {
        rs.sel[4 + 2 * r] = (b << 7) | (2 * lane + 1);
        rs.sel[5 + 2 * r] = (int32_t)(K - above);
      }
      above += c1;
      if (above < K && K <= above + c0) {
        rs.sel[4 + 2 * r] = (b << 7) | (2 * lane);
        rs.sel[5 + 2 * r] = (int32_t)(K - above);
      }
    }
  }
  __syncthreads();

  // 4. positions
  const uint32_t t1 = (uint32_t)rs.sel[4], q1 = (uint32_t)rs.sel[5];
  const uint32_t t2 = (uint32_t)rs.sel[6], q2 = (uint32_t)rs.sel[7];
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i >= nv) continue;
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    c[0] += k > t1;
    c[1] += k == t1;
    c[2] += k > t2;
    c[3] += k == t2;
  }
  uint32_t in[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) in[j] = wave_incl_scan(c[j]);
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rs.scan[j][wave] = in[j];
  }
  __syncthreads();
  uint32_t g1 = in[0] - c[0], e1r = in[1] - c[1], g2 = in[2] - c[2], e2r = in[3] - c[3];
  for (int w = 0; w < wave; ++w) {
    g1 += rs.scan[0][w];
    e1r += rs.scan[1][w];
    g2 += rs.scan[2][w];
    e2r += rs.scan[3][w];
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i >= nv) continue;
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool in_f = k > t1 || (k == t1 && e1r < q1);
    const bool in_fa = k > t2 || (k == t2 && e2r < q2);
    if (in_fa) {
      const int fpos = (int)(g1 + min(e1r, q1));          // F entries before this one
      const int apos = (int)(g2 + min(e2r, q2)) - fpos;   // A entries before this one
      const int j = base + i;
      int slot = -1;
      if (in_f && fpos >= f0 && fpos < f1) slot = fpos - f0;
      if (!in_f && apos >= a0 && apos < a1) slot = (f1 - f0) + (apos - a0);
      if (slot >= 0) {
        lidx[slot] = j;
        lx[slot] = h2f(rawbits(xr, i));
        if (write_lists) {
          if (in_f) a.out_full_idx[fpos] = j;
          else a.out_approx_idx[apos] = j;
        }
      }
    }
    g1 += k > t1;
    e1r += k == t1;
    g2 += k > t2;
    e2r += k == t2;
  }
  __syncthreads();
}

// Gate / up pair: r1 is a gate row, r1 + 128 the matching up row.
__device__ __forceinline__ void store_glu(const GemvArgs& a, int r1, float v1, float v2) {
  if (r1 < a.rows) {
    const int gi = (r1 >> 8) * 128 + (r1 & 127);
    const uint16_t gb = f2h(v1), ub = f2h(v2);
    const float g = h2f(gb), u = h2f(ub);
    const float sg = g / (1.0f + expf(-g));
    a.glu_a[gi] = f2h(sg * u);
    if (a.glu_g) a.glu_g[gi] = gb;
    if (a.glu_u) a.glu_u[gi] = ub;
  }
}

template <int FF, int AF, int MODE, int EPI, int E>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  // The rank scratch is dead once the list piece is in LDS; the wave
  // partials reuse it.
  union Scratch {
    RankShared rank;
    float red[kWaves][kTileRows];
  };
  __shared__ Scratch sm;
  __shared__ int32_t lidx[MODE == kListRank ? kListCap : 1];
  __shared__ float lx[MODE == kListRank ? kListCap : 1];
  __shared__ uint32_t last_flag;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int s_loc, tile;
  map_block(blockIdx.x, a.n_tiles, a.splits_here, s_loc, tile);
  const int split = a.split_lo + s_loc;
  const int row0 = tile * kTileRows;
  // Lanes past the last row of a ragged tile read lane 0's rows (in bounds);
  // their sums are never stored.
  const int ld_lane = row0 + 8 * lane < a.rows ? lane : 0;

  const int f0 = split_pos(split, a.n_splits, a.k_full);
  const int f1 = split_pos(split + 1, a.n_splits, a.k_full);
  const int a0 = split_pos(split, a.n_splits, a.k_approx);
  const int a1 = split_pos(split + 1, a.n_splits, a.k_approx);

  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  float corr = 0.0f;

  int f_lo, f_hi, a_lo, a_hi;  // tier ranges in the list (or in the LDS piece)
  if constexpr (MODE == kListRank) {
    // the piece holds F positions [f0, f1) then A positions [a0, a1)
    rank_piece<E>(a, sm.rank, lidx, lx, f0, f1, a0, a1, tile == 0);
    f_lo = 0;
    f_hi = f1 - f0;
    a_lo = f1 - f0;
    a_hi = f1 - f0 + a1 - a0;
  } else {
    f_lo = f0;
    f_hi = f1;
    a_lo = a0;
    a_hi = a1;
  }
  {
    const int lf = f_hi - f_lo, la = a_hi - a_lo;
    stream_tiers<FF, AF, MODE>(acc, corr, a, lidx, lx, f_lo + (lf * wave) / kWaves,
                               f_lo + (lf * (wave + 1)) / kWaves, a_lo + (la * wave) / kWaves,
                               a_lo + (la * (wave + 1)) / kWaves, row0, lane, ld_lane);
  }
  if constexpr (FF == kInt4 || AF != kNone) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] -= corr;
  }

  float4* dst = reinterpret_cast<float4*>(&sm.red[wave][8 * lane]);
  dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();

  // thread t owns row t of the tile from here on
  float p = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) p += sm.red[w][t];
  const int r = row0 + t;

  if (a.n_splits > 1) {
    // Cross-split reduction without cache-wide fences. The partials are
    // written and read with agent-scope relaxed atomics, which the gfx950
    // memory model maps to L2 write-through stores and L2-coherent loads,
    // so no L2 writeback or invalidate is needed: waiting for the stores
    // to complete before the counter increment orders them for every XCD.
    float* part = a.partials;
    const int64_t rows = a.rows;
    if (r < a.rows)
      __hip_atomic_store(&part[split * rows + r], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this lane's stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (t == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = old == (uint32_t)(a.n_splits - 1);
      if (last)
        __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = last;
    }
    __syncthreads();
    if (!last_flag) return;
    // partials are added in split order, 16 loads in flight
    p = 0.0f;
    const bool ok = r < a.rows;
    for (int s0 = 0; s0 < a.n_splits; s0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = (ok && s0 + u < a.n_splits)
                   ? __hip_atomic_load(&part[(s0 + u) * rows + r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < a.n_splits) p += v[u];
    }
  }

  if constexpr (EPI == kEpiPlain) {
    if (r < a.rows) a.y[r] = f2h(p);
  } else {
    __syncthreads();
    sm.red[0][t] = p;
    __syncthreads();
    if (t < kTileRows / 2) {
      const int i1 = (t >> 7) * 256 + (t & 127);
      store_glu(a, row0 + i1, sm.red[0][i1], sm.red[0][i1 + 128]);
    }
  }
}

template <int FF, int AF, int MODE, int E>
hipError_t launch_epi(const GemvArgs& a, int32_t epi, hipStream_t s) {
  const dim3 grid(a.n_tiles * a.splits_here), block(kGemvThreads);
  if (epi == kEpiGlu)
    hipLaunchKernelGGL((gemv_kernel<FF, AF, MODE, kEpiGlu, E>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<FF, AF, MODE, kEpiPlain, E>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int FF, int AF>
hipError_t launch_mode(const GemvArgs& a, int32_t mode, int32_t epi, hipStream_t s) {
  if (mode == kListStaged) return launch_epi<FF, AF, kListStaged, 0>(a, epi, s);
  if (mode == kListGlobal) return launch_epi<FF, AF, kListGlobal, 0>(a, epi, s);
  if (a.n <= kGemvThreads * 8) return launch_epi<FF, AF, kListRank, 8>(a, epi, s);
  if (a.n <= kGemvThreads * 16) return launch_epi<FF, AF, kListRank, 16>(a, epi, s);
  if (a.n <= kGemvThreads * 32) return launch_epi<FF, AF, kListRank, 32>(a, epi, s);
  if (a.n <= kGemvThreads * 64) return launch_epi<FF, AF, kListRank, 64>(a, epi, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, int32_t full_fmt, int32_t approx_fmt, int32_t mode,
                       int32_t epi, hipStream_t s) {
  if (full_fmt == kFp16) {
    if (approx_fmt == kNone) return launch_mode<kFp16, kNone>(a, mode, epi, s);
    if (approx_fmt == kInt4) return launch_mode<kFp16, kInt4>(a, mode, epi, s);
    if (approx_fmt == kInt2) return launch_mode<kFp16, kInt2>(a, mode, epi, s);
  } else if (full_fmt == kInt4) {
    if (approx_fmt == kNone) return launch_mode<kInt4, kNone>(a, mode, epi, s);
    if (approx_fmt == kInt4) return launch_mode<kInt4, kInt4>(a, mode, epi, s);
    if (approx_fmt == kInt2) return launch_mode<kInt4, kInt2>(a, mode, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spax
