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
  static __device__ __forceinline__ void fma(float (&acc)[8], float&, V v, float xs, uint32_t) {
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
                                             uint32_t scale) {
    const float c = xs * h2f(scale);  // exact: product of two fp16 values
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
                                             uint32_t scale) {
    const float c = xs * h2f(scale);
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

// Stream list positions [p_lo, p_hi) of one tier for this wave's rows.
//   kListGlobal: idx = global index list, x = global fp16 activations;
//   kListStaged: idx = global index list (for x only), column = position;
//   kListRank:   lidx / lx = this workgroup's list piece in LDS (index and
//                fp32 activation per position).
template <int FMT, int MODE>
__device__ __forceinline__ void run_tier(float (&acc)[8], float& corr,
                                         const uint8_t* __restrict__ base, int64_t stride,
                                         const uint16_t* __restrict__ scales, int64_t sstride,
                                         const int32_t* __restrict__ idx,
                                         const uint16_t* __restrict__ x, const int32_t* lidx,
                                         const float* lx, int p_lo, int p_hi, int row0, int lane,
                                         int ld_lane) {
  // lane: this lane's slot in the 64-wide batches of indices / activations;
  // ld_lane: the lane whose rows it loads (lane 0 past the last row)
  using T = Tier<FMT>;
  constexpr int U = T::U;
  const int sc_off = (row0 >> 7) + (ld_lane >> 4);
  int nxt = 0;
  if constexpr (MODE != kListRank) {
    if (p_lo < p_hi && lane < p_hi - p_lo) nxt = idx[p_lo + lane];
  }
  for (int kb = p_lo; kb < p_hi; kb += 64) {
    const int cnt = min(64, p_hi - kb);
    int my_idx;
    uint32_t my_xb;  // fp16 bits (global modes) or fp32 bits (rank mode)
    if constexpr (MODE == kListRank) {
      const int q = lane < cnt ? kb + lane : kb;
      my_idx = lidx[q];
      my_xb = __float_as_uint(lx[q]);
    } else {
      my_idx = nxt;
      // prefetch the next batch of indices before streaming this one
      if (kb + 64 < p_hi && lane < p_hi - kb - 64) nxt = idx[kb + 64 + lane];
      // raw fp16 bits; converted where used so that this gather overlaps the
      // weight loads (lanes >= cnt hold an in-range stale index, never read)
      my_xb = x[my_idx];
    }
    auto xval = [&](int c) -> float {
      const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)my_xb, c);
      if constexpr (MODE == kListRank) return __uint_as_float(b);
      else return h2f(b);
    };
    int c = 0;
    for (; c + U <= cnt; c += U) {
      typename T::V v[U];
      uint32_t sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = MODE == kListStaged ? (kb + c + u)
                                            : __builtin_amdgcn_readlane(my_idx, c + u);
        const uint8_t* cp = base + (int64_t)col * stride;
        v[u] = T::load(cp, row0, ld_lane);
        if constexpr (FMT != kFp16)
          sv[u] = scales[(int64_t)col * sstride + sc_off];
        else
          sv[u] = 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) T::fma(acc, corr, v[u], xval(c + u), sv[u]);
    }
    for (; c < cnt; ++c) {
      const int col = MODE == kListStaged ? (kb + c) : __builtin_amdgcn_readlane(my_idx, c);
      const uint8_t* cp = base + (int64_t)col * stride;
      const typename T::V v = T::load(cp, row0, ld_lane);
      uint32_t sv = 0u;
      if constexpr (FMT != kFp16) sv = scales[(int64_t)col * sstride + sc_off];
      T::fma(acc, corr, v, xval(c), sv);
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

__device__ __forceinline__ uint32_t wave_excl_suffix(uint32_t v, int lane) {
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_down(incl, d, 64);
    if (lane + d < 64) incl += t;
  }
  return incl - v;
}

__device__ __forceinline__ uint32_t rawbits(const uint32_t* xr, int i) {
  return (xr[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

// Ranks x and places this workgroup's list positions [e0, e1) in LDS.
// Returns the number of full-tier positions in the piece.
template <int E>
__device__ __forceinline__ int rank_piece(const GemvArgs& a, RankShared& rs, int32_t* lidx,
                                          float* lx, int64_t e0, int64_t e1, bool write_lists) {
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
    uint32_t above = wave_excl_suffix(c[0] + c[1] + c[2] + c[3], lane);
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
      uint32_t above = (uint32_t)rs.sel[1 + 2 * r] + wave_excl_suffix(c0 + c1, lane);
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
  uint32_t in[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = __shfl_up(in[j], d, 64);
      if (lane >= d) in[j] += v;
    }
  }
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
  const int kf = a.k_full;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i >= nv) continue;
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool in_f = k > t1 || (k == t1 && e1r < q1);
    const bool in_fa = k > t2 || (k == t2 && e2r < q2);
    if (in_fa) {
      const int64_t fpos = g1 + min(e1r, q1);          // F entries before this one
      const int64_t apos = g2 + min(e2r, q2) - fpos;   // A entries before this one
      const int64_t v = in_f ? fpos : kf + apos;
      const int j = base + i;
      if (v >= e0 && v < e1) {
        lidx[v - e0] = j;
        lx[v - e0] = h2f(rawbits(xr, i));
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
  return (int)(min<int64_t>(e1, kf) - min<int64_t>(e0, kf));
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

  const int64_t e0 = split_start(split, a.n_splits, a.k_full, a.k_approx, a.w_full, a.w_approx);
  const int64_t e1 = split_start(split + 1, a.n_splits, a.k_full, a.k_approx, a.w_full, a.w_approx);

  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  float corr = 0.0f;

  int f_lo, f_hi, a_lo, a_hi;  // tier ranges in the list (or in the LDS piece)
  if constexpr (MODE == kListRank) {
    const int nf = rank_piece<E>(a, sm.rank, lidx, lx, e0, e1, tile == 0);
    f_lo = 0;
    f_hi = nf;
    a_lo = nf;
    a_hi = (int)(e1 - e0);
  } else {
    f_lo = (int)min<int64_t>(e0, a.k_full);
    f_hi = (int)min<int64_t>(e1, a.k_full);
    a_lo = (int)(max<int64_t>(e0, a.k_full) - a.k_full);
    a_hi = (int)(max<int64_t>(e1, a.k_full) - a.k_full);
  }
  {
    const int len = f_hi - f_lo;
    const int wlo = f_lo + (len * wave) / kWaves, whi = f_lo + (len * (wave + 1)) / kWaves;
    run_tier<FF, MODE>(acc, corr, a.full_base, a.full_stride, a.full_scales, a.full_sstride,
                       a.full_idx, a.x, lidx, lx, wlo, whi, row0, lane, ld_lane);
  }
  if constexpr (AF != kNone) {
    const int len = a_hi - a_lo;
    const int wlo = a_lo + (len * wave) / kWaves, whi = a_lo + (len * (wave + 1)) / kWaves;
    run_tier<AF, MODE>(acc, corr, a.approx_base, a.approx_stride, a.approx_scales,
                       a.approx_sstride, a.approx_idx, a.x, lidx, lx, wlo, whi, row0, lane,
                       ld_lane);
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
