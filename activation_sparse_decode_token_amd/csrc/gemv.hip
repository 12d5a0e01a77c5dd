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

// Buffer resource of one tier of a matrix: a scalar base and size. A
// column's load adds the column offset as the 32-bit scalar soffset and the
// lane's part as one shared 32-bit vector offset, so each load costs one
// scalar register instead of a 64-bit address per lane. Reads past the tier
// return 0 instead of touching memory. Dword 3 selects 32-bit raw access on
// gfx9-family parts. Tier sizes are below 2^31 bytes (checked on the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tier_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

template <int FMT>
struct Tier;

// Opaque to the optimiser: keeps the byte-wise code extraction below from
// being folded into per-value bit-field extracts, so each value is one
// v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <>
struct Tier<kFp16> {
  using V = uint4;
  static constexpr int U = 8;
  // byte offset of lane l's 8 rows in a column
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return 2u * (uint32_t)(row0 + 8 * lane);
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t, off, col, 0));
  }
  // f = x_j
  static __device__ __forceinline__ void fma(float (&acc)[8], float&, V v, float f) {
    acc[0] = fmaf(h2f(v.x & 0xFFFFu), f, acc[0]);
    acc[1] = fmaf(h2f(v.x >> 16), f, acc[1]);
    acc[2] = fmaf(h2f(v.y & 0xFFFFu), f, acc[2]);
    acc[3] = fmaf(h2f(v.y >> 16), f, acc[3]);
    acc[4] = fmaf(h2f(v.z & 0xFFFFu), f, acc[4]);
    acc[5] = fmaf(h2f(v.z >> 16), f, acc[5]);
    acc[6] = fmaf(h2f(v.w & 0xFFFFu), f, acc[6]);
    acc[7] = fmaf(h2f(v.w >> 16), f, acc[7]);
  }
};

template <>
struct Tier<kInt4> {
  using V = uint32_t;
  static constexpr int U = 16;
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 2u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_amdgcn_raw_buffer_load_b32(t, off, col, 0);
  }
  // Rows 2b and 2b+1 sit in the low and high nibble of byte b, as
  // two's-complement q; flipping each nibble's sign bit gives u = q + 8.
  // f = x_j * s_{j,g} (exact: a product of two fp16 values); the offset 8 f
  // is taken off through corr.
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float f) {
    corr = fmaf(8.0f, f, corr);
    v ^= 0x88888888u;
    const uint32_t lo = opaque(v & 0x0F0F0F0Fu);
    const uint32_t hi = opaque((v >> 4) & 0x0F0F0F0Fu);
    acc[0] = fmaf(f, b2f(lo, 0), acc[0]);
    acc[1] = fmaf(f, b2f(hi, 0), acc[1]);
    acc[2] = fmaf(f, b2f(lo, 1), acc[2]);
    acc[3] = fmaf(f, b2f(hi, 1), acc[3]);
    acc[4] = fmaf(f, b2f(lo, 2), acc[4]);
    acc[5] = fmaf(f, b2f(hi, 2), acc[5]);
    acc[6] = fmaf(f, b2f(lo, 3), acc[6]);
    acc[7] = fmaf(f, b2f(hi, 3), acc[7]);
  }
};

template <>
struct Tier<kInt2> {
  using V = uint32_t;
  static constexpr int U = 16;
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 4u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_amdgcn_raw_buffer_load_b16(t, off, col, 0);
  }
  // Row 4b + r sits in bits 2r..2r+1 of byte b (two bytes per lane); each
  // 2-bit field is moved to the bottom of its byte and converted. The
  // offset 1.5 f is taken off through corr.
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float f) {
    corr = fmaf(1.5f, f, corr);
    const uint32_t m0 = opaque(v & 0x0303u);
    const uint32_t m1 = opaque((v >> 2) & 0x0303u);
    const uint32_t m2 = opaque((v >> 4) & 0x0303u);
    const uint32_t m3 = opaque((v >> 6) & 0x0303u);
    acc[0] = fmaf(f, b2f(m0, 0), acc[0]);
    acc[4] = fmaf(f, b2f(m0, 1), acc[4]);
    acc[1] = fmaf(f, b2f(m1, 0), acc[1]);
    acc[5] = fmaf(f, b2f(m1, 1), acc[5]);
    acc[2] = fmaf(f, b2f(m2, 0), acc[2]);
    acc[6] = fmaf(f, b2f(m2, 1), acc[6]);
    acc[3] = fmaf(f, b2f(m3, 0), acc[3]);
    acc[7] = fmaf(f, b2f(m3, 1), acc[7]);
  }
};

// Metadata of one wave's current 64-column batch of one tier, in LDS: the
// column (stored index, or staging position) and the factor each lane
// multiplies that column by -- x_j for fp16 columns, x_j * s_{j,g} for code
// columns, one per 128-row group g of the tile.
struct WaveMeta {
  int32_t col[64];
  float fac[64][4];
};

// Fill the batch's metadata: lane l takes batch position p + l.
//   kListGlobal: idx = global index list, x = global fp16 activations;
//   kListStaged: column = list position (staging), x via the index list;
//   kListRank:   lidx / lx = this workgroup's list piece in LDS.
template <int FMT, int MODE>
__device__ __forceinline__ void fill_meta(WaveMeta& wm, const uint16_t* __restrict__ scales,
                                          int64_t sstride, const int32_t* __restrict__ idx,
                                          const uint16_t* __restrict__ x, const int32_t* lidx,
                                          const float* lx, int p, int cnt, int row0, int ngrp,
                                          int lane) {
  if (lane < cnt) {
    const int q = p + lane;
    int j;
    float xv;
    if constexpr (MODE == kListRank) {
      j = lidx[q];
      xv = lx[q];
    } else {
      j = idx[q];
      xv = h2f(x[j]);
    }
    const int col = MODE == kListStaged ? q : j;
    wm.col[lane] = col;
    if constexpr (FMT == kFp16) {
      wm.fac[lane][0] = xv;
    } else {
      // a ragged last tile has fewer groups; their slots are never read
      // (lanes past the last row take group 0's rows)
      const uint16_t* sp = scales + (int64_t)col * sstride + (row0 >> 7);
      const int gl = ngrp - 1;
#pragma unroll
      for (int g = 0; g < 4; ++g) wm.fac[lane][g] = xv * h2f(sp[min(g, gl)]);
    }
  }
  // the batch's slots are read by every lane of this wave below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stream this wave's list positions [p_lo, p_hi) of one tier for its rows.
// Rounds of U columns are double-buffered: the loads of round r + 1 are
// issued before round r is consumed, so a wave always has a round in flight.
// Each step issues and consumes in one straight-line block (the wait before
// the consumption counts only the loads issued just before it). Slots past
// the batch reload its last column and add it times zero, which keeps every
// load unconditional.
template <int FMT, int MODE>
__device__ __forceinline__ void stream_tier(float (&acc)[8], float& corr, WaveMeta& wm,
                                            const uint8_t* base, int64_t stride, uint32_t bytes,
                                            const uint16_t* scales, int64_t sstride,
                                            const int32_t* idx, const uint16_t* x,
                                            const int32_t* lidx, const float* lx, int p_lo,
                                            int p_hi, int row0, int rows, int lane,
                                            int ld_lane) {
  using T = Tier<FMT>;
  constexpr int U = T::U;
  constexpr bool kCode = FMT != kFp16;
  const int gsel = kCode ? (ld_lane >> 4) : 0;  // this lane's group in the tile
  const int ngrp = min(4, (rows - row0 + kGroup - 1) / kGroup);
  const uint32_t off = T::offset(row0, ld_lane);
  const __amdgpu_buffer_rsrc_t rs = tier_rsrc(base, bytes);
  const uint32_t cstride = (uint32_t)stride;
  for (int pb = p_lo; pb < p_hi; pb += 64) {
    const int cnt = min(64, p_hi - pb);
    fill_meta<FMT, MODE>(wm, scales, sstride, idx, x, lidx, lx, pb, cnt, row0, ngrp, lane);
    const int rounds = (cnt + U - 1) / U;
    typename T::V v0[U], v1[U];
    auto issue = [&](int r, typename T::V (&v)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(r * U + u, cnt - 1);
        const uint32_t col = (uint32_t)__builtin_amdgcn_readfirstlane(wm.col[c]);
        v[u] = T::load(rs, off, col * cstride);
      }
    };
    auto use = [&](int r, const typename T::V (&v)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = r * U + u;
        const float f = c < cnt ? wm.fac[c][gsel] : 0.0f;
        T::fma(acc, corr, v[u], f);
      }
    };
    issue(0, v0);
    for (int r = 0;;) {
      if (r + 1 < rounds) {
        issue(r + 1, v1);
        use(r, v0);
      } else {
        use(r, v0);
        break;
      }
      ++r;
      if (r + 1 < rounds) {
        issue(r + 1, v0);
        use(r, v1);
      } else {
        use(r, v1);
        break;
      }
      ++r;
    }
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
  __shared__ WaveMeta wmeta[kWaves];
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
    WaveMeta& wm = wmeta[wave];
    const int lf = f_hi - f_lo, la = a_hi - a_lo;
    stream_tier<FF, MODE>(acc, corr, wm, a.full_base, a.full_stride, a.full_bytes,
                          a.full_scales, a.full_sstride, a.full_idx, a.x, lidx, lx,
                          f_lo + (lf * wave) / kWaves, f_lo + (lf * (wave + 1)) / kWaves, row0,
                          a.rows, lane, ld_lane);
    if constexpr (AF != kNone)
      stream_tier<AF, MODE>(acc, corr, wm, a.approx_base, a.approx_stride, a.approx_bytes,
                            a.approx_scales, a.approx_sstride, a.approx_idx, a.x, lidx, lx,
                            a_lo + (la * wave) / kWaves, a_lo + (la * (wave + 1)) / kWaves, row0,
                            a.rows, lane, ld_lane);
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
