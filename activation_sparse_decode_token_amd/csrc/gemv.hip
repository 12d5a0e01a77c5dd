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

// Buffer resource of one column: a wave-uniform base in scalar registers
// (pinned with readfirstlane so no lane offset is folded into it). Loads
// through it take one shared 32-bit lane offset instead of a 64-bit address
// per lane and load. Dword 3 selects 32-bit raw access on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t column_rsrc(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7FFFFFFF, 0x00020000);
}

template <int FMT>
struct Tier;

template <>
struct Tier<kFp16> {
  using V = uint4;
  static constexpr int U = 8;
  // byte offset of lane l's 8 rows in a column
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return 2u * (uint32_t)(row0 + 8 * lane);
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t col, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(col, off, 0, 0));
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
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 2u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t col, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(col, off, 0, 0);
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
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 4u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t col, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(col, off, 0, 0);
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
  uint32_t g[4];  // raw scales as loaded (code tiers)
  uint32_t sc01, sc23;  // packed by pack_scales once the round's loads are issued
};

template <int FMT, int MODE>
__device__ __forceinline__ Meta load_meta(const uint16_t* __restrict__ scales, int64_t sstride,
                                          const int32_t* __restrict__ idx,
                                          const uint16_t* __restrict__ x, const int32_t* lidx,
                                          const float* lx, int p, int cnt, int row0, int ngrp,
                                          int lane) {
  Meta m{0, 0u, {0u, 0u, 0u, 0u}, 0u, 0u};
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
    // a ragged last tile has fewer groups: their slots repeat its last group
    // (never used, since lanes past the last row take group 0's rows), so
    // the four loads are unconditional and issue back to back
    const int64_t col = MODE == kListStaged ? (int64_t)q : (int64_t)m.idx;
    const uint16_t* sp = scales + col * sstride + (row0 >> 7);
    const int gl = ngrp - 1;
    m.g[0] = sp[0];
    m.g[1] = sp[min(1, gl)];
    m.g[2] = sp[min(2, gl)];
    m.g[3] = sp[min(3, gl)];
  }
  return m;
}

__device__ __forceinline__ void pack_scales(Meta& m) {
  // The empty volatile asm makes the raw scales opaque, so the packing (which
  // waits for the scale loads) is not hoisted out of the round loop ahead of
  // the round's weight loads.
  asm volatile("" : "+v"(m.g[0]), "+v"(m.g[1]), "+v"(m.g[2]), "+v"(m.g[3]));
  m.sc01 = m.g[0] | (m.g[1] << 16);
  m.sc23 = m.g[2] | (m.g[3] << 16);
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
template <typename T, int U, int MODE, bool CODE>
__device__ __forceinline__ void consume(float (&acc)[8], float& corr, const typename T::V (&v)[U],
                                        const Meta& m, int c0, int n, bool hi_pair, uint32_t sh) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + (u < n ? u : 0);
    const float xs = u < n ? meta_x<MODE>(m, c) : 0.0f;
    const float sc = CODE ? meta_scale(m, c, hi_pair, sh) : 0.0f;
    T::fma(acc, corr, v[u], xs, sc);
  }
}

// Stream this wave's full-tier list positions [f_lo, f_hi) and approx-tier
// positions [a_lo, a_hi) for its rows. Each round issues the loads of UF
// full columns and UA code columns before any of them is consumed, so a wave
// keeps both tiers' bytes in flight together. Slots past a tier's share
// reload a valid column and add it times zero, which keeps every load
// unconditional: the compiler then issues a round's loads back to back.
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
  constexpr bool kHasA = AF != kNone;
  constexpr int UF = TF::U;
  // equal rounds for equal column counts when the full tier is fp16
  constexpr int UA = FF == kFp16 ? 8 : TA::U;
  const int grp = ld_lane >> 4;  // this lane's group in the tile
  const bool hi_pair = grp >= 2;
  const uint32_t sh = 16u * (uint32_t)(grp & 1);
  const int ngrp = min(4, (a.rows - row0 + kGroup - 1) / kGroup);
  // column bases are wave-uniform (buffer resources in scalar registers);
  // the lane's part of the address is one 32-bit offset per tier
  const uint32_t off_f = TF::offset(row0, ld_lane);
  const uint32_t off_a = TA::offset(row0, ld_lane);
  if constexpr (!kHasA) a_hi = a_lo;
  int pf = f_lo, pa = a_lo;
  while (pf < f_hi || pa < a_hi) {
    const int nbf = max(0, min(64, f_hi - pf)), nba = max(0, min(64, a_hi - pa));
    Meta mf = load_meta<FF, MODE>(a.full_scales, a.full_sstride, a.full_idx, a.x, lidx, lx, pf,
                                  nbf, row0, ngrp, lane);
    Meta ma{0, 0u, {0u, 0u, 0u, 0u}, 0u, 0u};
    if constexpr (kHasA)
      ma = load_meta<AF, MODE>(a.approx_scales, a.approx_sstride, a.approx_idx, a.x, lidx, lx,
                               pa, nba, row0, ngrp, lane);
    const int rounds = max((nbf + UF - 1) / UF, kHasA ? (nba + UA - 1) / UA : 0);
    // Double-buffered rounds: the loads of round r + 1 are issued before
    // round r is consumed, so a wave always has a round in flight. Each step
    // issues and consumes in one straight-line block, so the wait before the
    // consumption counts only the loads issued just before it.
    typename TF::V vf0[UF], vf1[UF];
    typename TA::V va0[kHasA ? UA : 1], va1[kHasA ? UA : 1];
    auto issue = [&](int r, typename TF::V (&vf)[UF], typename TA::V (&va)[kHasA ? UA : 1]) {
      const int cf = r * UF, ca = r * UA;
      const int nf = min(UF, nbf - cf), na = min(UA, nba - ca);
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        // an exhausted tier reloads a valid column of its batch
        const int c = min(cf + (u < nf ? u : 0), 63);
        vf[u] = TF::load(
            column_rsrc(a.full_base + (int64_t)meta_col<MODE>(mf, pf, c) * a.full_stride), off_f);
      }
      if constexpr (kHasA) {
#pragma unroll
        for (int u = 0; u < UA; ++u) {
          const int c = min(ca + (u < na ? u : 0), 63);
          va[u] = TA::load(
              column_rsrc(a.approx_base + (int64_t)meta_col<MODE>(ma, pa, c) * a.approx_stride),
              off_a);
        }
      }
      // keep the scale packing (which waits for the scale loads) behind the
      // weight loads so the two round trips overlap
      __builtin_amdgcn_sched_barrier(0);
    };
    auto use = [&](int r, const typename TF::V (&vf)[UF],
                   const typename TA::V (&va)[kHasA ? UA : 1]) {
      const int cf = r * UF, ca = r * UA;
      const int nf = min(UF, nbf - cf), na = min(UA, nba - ca);
      if constexpr (FF != kFp16) pack_scales(mf);
      if constexpr (kHasA) pack_scales(ma);
      consume<TF, UF, MODE, FF != kFp16>(acc, corr, vf, mf, cf, nf, hi_pair, sh);
      if constexpr (kHasA) consume<TA, UA, MODE, true>(acc, corr, va, ma, ca, na, hi_pair, sh);
    };
    if (rounds > 0) {
      issue(0, vf0, va0);
      for (int r = 0;;) {
        if (r + 1 < rounds) {
          issue(r + 1, vf1, va1);
          use(r, vf0, va0);
        } else {
          use(r, vf0, va0);
          break;
        }
        ++r;
        if (r + 1 < rounds) {
          issue(r + 1, vf0, va0);
          use(r, vf1, va1);
        } else {
          use(r, vf1, va1);
          break;
        }
        ++r;
      }
    }
    pf += nbf;
    pa += nba;
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
//   1. 256-bin histogram of key bits 14..7 (LDS atomics);
//   2. suffix counts give the bins holding rank k_full and k_full + k_approx;
//   3. 128-bin histograms inside those bins give the boundary keys t1, t2
//      and the number of entries equal to each that are kept (q1, q2);
//   4. one block scan of (#key > t1, #key == t1, #key > t2, #key == t2) gives
//      every entry its position: #F before entry i is
//      gt1(i) + min(eq1(i), q1), #(F or A) before it gt2(i) + min(eq2(i), q2).
// ---------------------------------------------------------------------------
constexpr uint32_t kAboveAll = 0x8000u;  // boundary key when a tier is empty

struct RankShared {
  uint32_t hist[257];  // bin 256 absorbs the padding past n
  uint32_t sub[2][128];
  uint32_t scan[4][kWaves];
  int32_t sel[8];  // b1, entries above b1, b2, entries above b2, t1, q1, t2, q2
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

// The one lane with sel >= 0 (if any) broadcasts (sel, val) to the wave;
// otherwise out_sel = -1, out_val = 0.
__device__ __forceinline__ void wave_pick(int sel, uint32_t val, int& out_sel,
                                          uint32_t& out_val) {
  const uint64_t m = __ballot(sel >= 0);
  if (m == 0) {
    out_sel = -1;
    out_val = 0u;
  } else {
    const int src = (int)__builtin_ctzll(m);
    out_sel = __builtin_amdgcn_readlane(sel, src);
    out_val = (uint32_t)__builtin_amdgcn_readlane((int)val, src);
  }
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

  if (t < 256) {
    rs.hist[t] = 0u;
    (&rs.sub[0][0])[t] = 0u;
  }
  if (t == 256) rs.hist[256] = 0u;
  __syncthreads();

  // 1. top-level histogram
#pragma unroll
  for (int i = 0; i < E; ++i)
    atomicAdd(&rs.hist[i < nv ? (rawbits(xr, i) & 0x7FFFu) >> 7 : 256u], 1u);
  __syncthreads();

  // 2. bins holding rank K1 and rank K2 (1-based, from the largest key),
  // found by wave 0 (the other waves wait at the barrier, leaving it the
  // whole SIMD)
  if (wave == 0) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = rs.hist[4 * lane + j];
    uint32_t above = wave_excl_suffix(c[0] + c[1] + c[2] + c[3]);
    int s1 = -1, s2 = -1;
    uint32_t x1 = 0u, x2 = 0u;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (K1 > 0 && above < K1 && K1 <= above + c[j]) { s1 = 4 * lane + j; x1 = above; }
      if (K2 > 0 && above < K2 && K2 <= above + c[j]) { s2 = 4 * lane + j; x2 = above; }
      above += c[j];
    }
    int b, ab;
    uint32_t v;
    wave_pick(s1, x1, b, v);
    ab = (int)v;
    if (lane == 0) { rs.sel[0] = b; rs.sel[1] = ab; }
    wave_pick(s2, x2, b, v);
    ab = (int)v;
    if (lane == 0) { rs.sel[2] = b; rs.sel[3] = ab; }
  }
  __syncthreads();

  // 3. low-level histograms inside the two boundary bins
  const int b1 = rs.sel[0];
  const int b2 = rs.sel[2];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const int hb = i < nv ? (int)(k >> 7) : 256;
    if (hb == b1) atomicAdd(&rs.sub[0][k & 127u], 1u);
    if (hb == b2) atomicAdd(&rs.sub[1][k & 127u], 1u);
  }
  __syncthreads();
  // boundary keys t (kAboveAll when the tier is empty) and quotas q: the
  // number of entries equal to t that are kept; found by wave 0
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = r == 0 ? b1 : b2;
      const uint32_t K = r == 0 ? K1 : K2;
      int key = (int)kAboveAll;
      uint32_t quota = 0u;
      if (b >= 0) {  // wave-uniform
        const uint32_t c0 = rs.sub[r][2 * lane], c1 = rs.sub[r][2 * lane + 1];
        uint32_t above = (uint32_t)rs.sel[1 + 2 * r] + wave_excl_suffix(c0 + c1);
        int sk = -1;
        uint32_t sq = 0u;
        if (above < K && K <= above + c1) { sk = (b << 7) | (2 * lane + 1); sq = K - above; }
        above += c1;
        if (above < K && K <= above + c0) { sk = (b << 7) | (2 * lane); sq = K - above; }
        wave_pick(sk, sq, key, quota);
      }
      if (lane == 0) {
        rs.sel[4 + 2 * r] = key;
        rs.sel[5 + 2 * r] = (int32_t)quota;
      }
    }
  }
  __syncthreads();
  const uint32_t t1 = (uint32_t)rs.sel[4], q1 = (uint32_t)rs.sel[5];
  const uint32_t t2 = (uint32_t)rs.sel[6], q2 = (uint32_t)rs.sel[7];

  // 4. positions
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool ok = i < nv;
    c[0] += ok && k > t1;
    c[1] += ok && k == t1;
    c[2] += ok && k > t2;
    c[3] += ok && k == t2;
  }
  uint32_t in[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) in[j] = wave_incl_scan(c[j]);
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rs.scan[j][wave] = in[j];
  }
  __syncthreads();
  // totals of the waves before this one: lanes 0..7 hold the wave totals,
  // a lane scan gives their prefixes, lane `wave` holds this wave's
  uint32_t pre[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t wt = lane < kWaves ? rs.scan[j][lane] : 0u;
    pre[j] = (uint32_t)__builtin_amdgcn_readlane((int)(wave_incl_scan(wt) - wt), wave);
  }
  uint32_t g1 = pre[0] + in[0] - c[0], e1r = pre[1] + in[1] - c[1];
  uint32_t g2 = pre[2] + in[2] - c[2], e2r = pre[3] + in[3] - c[3];
  // This thread's F positions [fs, fe) and A positions [as, ae); only
  // threads whose positions meet the piece place entries.
  const int fs = (int)(g1 + min(e1r, q1));
  const int fe = (int)(g1 + c[0] + min(e1r + c[1], q1));
  const int as = (int)(g2 + min(e2r, q2)) - fs;
  const int ae = (int)(g2 + c[2] + min(e2r + c[3], q2)) - fe;
  if ((fs < f1 && fe > f0) || (as < a1 && ae > a0)) {
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
    // partials are added in split order; the loads of up to 32 splits are
    // issued together (clamped to valid addresses, unused ones not added)
    p = 0.0f;
    const int64_t rr = min(r, a.rows - 1);
    for (int s0 = 0; s0 < a.n_splits; s0 += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        v[u] = __hip_atomic_load(&part[(int64_t)min(s0 + u, a.n_splits - 1) * rows + rr],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 32; ++u)
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
