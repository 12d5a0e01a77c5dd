// Tiered gather-GEMV (gfx950).
//
// SpAx page, section 2 Eq. 1 and section 5, Figure 2 steps 4-5:
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
//     piece for its tile; its 4 waves take contiguous quarters of the piece.
//   * Column indices and activations are fetched 64 at a time (one per lane)
//     and broadcast with readlane, so column addresses are wave-uniform.
//   * Code tiers fold x_j * s_{j,g} into one fp32 factor per column and lane
//     and accumulate the unsigned code; the code offset (8 for int4, 1.5 for
//     int2) is removed once at the end through a per-lane running sum.
//   * The 4 wave partials are added in LDS in a fixed order. With one split
//     the workgroup writes y; otherwise each workgroup stores its fp32 partial
//     and the last workgroup of a tile (agent-scope counter) adds the n_splits
//     partials in split order and writes y. The counter is reset by that
//     workgroup. The summation order never depends on timing, so results are
//     bitwise reproducible.
//   * The tiles of one split run on one XCD (blocks are dealt to the 8 XCDs
//     round-robin), so the shared index/activation/scale lines of a split hit
//     that XCD's L2.
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
template <int FMT, bool STAGED>
__device__ __forceinline__ void run_tier(float (&acc)[8], float& corr,
                                         const uint8_t* __restrict__ base, int64_t stride,
                                         const uint16_t* __restrict__ scales, int64_t sstride,
                                         const int32_t* __restrict__ idx,
                                         const uint16_t* __restrict__ x, int p_lo, int p_hi,
                                         int row0, int lane, int ld_lane) {
  // lane: this lane's slot in the 64-wide batches of indices / activations;
  // ld_lane: the lane whose rows it loads (lane 0 past the last row)
  using T = Tier<FMT>;
  constexpr int U = T::U;
  const int sc_off = (row0 >> 7) + (ld_lane >> 4);
  int nxt = 0;
  if (p_lo < p_hi && lane < p_hi - p_lo) nxt = idx[p_lo + lane];
  for (int kb = p_lo; kb < p_hi; kb += 64) {
    const int cnt = min(64, p_hi - kb);
    const int my_idx = nxt;
    // prefetch the next batch of indices before streaming this one
    if (kb + 64 < p_hi && lane < p_hi - kb - 64) nxt = idx[kb + 64 + lane];
    // raw fp16 bits; converted where used so that this gather overlaps the
    // weight loads (lanes >= cnt hold an in-range stale index, never read)
    const uint32_t my_xb = x[my_idx];
    int c = 0;
    for (; c + U <= cnt; c += U) {
      typename T::V v[U];
      uint32_t sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = STAGED ? (kb + c + u) : __builtin_amdgcn_readlane(my_idx, c + u);
        const uint8_t* cp = base + (int64_t)col * stride;
        v[u] = T::load(cp, row0, ld_lane);
        if constexpr (FMT != kFp16)
          sv[u] = scales[(int64_t)col * sstride + sc_off];
        else
          sv[u] = 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float xs = h2f((uint32_t)__builtin_amdgcn_readlane((int)my_xb, c + u));
        T::fma(acc, corr, v[u], xs, sv[u]);
      }
    }
    for (; c < cnt; ++c) {
      const int col = STAGED ? (kb + c) : __builtin_amdgcn_readlane(my_idx, c);
      const uint8_t* cp = base + (int64_t)col * stride;
      const typename T::V v = T::load(cp, row0, ld_lane);
      uint32_t sv = 0u;
      if constexpr (FMT != kFp16) sv = scales[(int64_t)col * sstride + sc_off];
      const float xs = h2f((uint32_t)__builtin_amdgcn_readlane((int)my_xb, c));
      T::fma(acc, corr, v, xs, sv);
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

template <int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int r1, int r2, float v1, float v2) {
  if constexpr (EPI == kEpiPlain) {
    if (r1 < a.rows) a.y[r1] = f2h(v1);
    if (r2 < a.rows) a.y[r2] = f2h(v2);
  } else {
    // r1 is a gate row, r2 = r1 + 128 the matching up row
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
}

template <int FF, int AF, bool STAGED, int EPI>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  __shared__ float red[kWaves][kTileRows];
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

  {
    const int lo = (int)min<int64_t>(e0, a.k_full), hi = (int)min<int64_t>(e1, a.k_full);
    const int len = hi - lo;
    const int wlo = lo + (len * wave) / kWaves, whi = lo + (len * (wave + 1)) / kWaves;
    run_tier<FF, STAGED>(acc, corr, a.full_base, a.full_stride, a.full_scales, a.full_sstride,
                         a.full_idx, a.x, wlo, whi, row0, lane, ld_lane);
  }
  if constexpr (AF != kNone) {
    const int lo = (int)(max<int64_t>(e0, a.k_full) - a.k_full);
    const int hi = (int)(max<int64_t>(e1, a.k_full) - a.k_full);
    const int len = hi - lo;
    const int wlo = lo + (len * wave) / kWaves, whi = lo + (len * (wave + 1)) / kWaves;
    run_tier<AF, STAGED>(acc, corr, a.approx_base, a.approx_stride, a.approx_scales,
                         a.approx_sstride, a.approx_idx, a.x, wlo, whi, row0, lane, ld_lane);
  }
  if constexpr (FF == kInt4 || AF != kNone) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] -= corr;
  }

  float4* dst = reinterpret_cast<float4*>(&red[wave][8 * lane]);
  dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();

  const int i1 = (t >> 7) * 256 + (t & 127);
  const int i2 = i1 + 128;
  const float p1 = ((red[0][i1] + red[1][i1]) + red[2][i1]) + red[3][i1];
  const float p2 = ((red[0][i2] + red[1][i2]) + red[2][i2]) + red[3][i2];
  const int r1 = row0 + i1, r2 = row0 + i2;

  if (a.n_splits == 1) {
    epilogue<EPI>(a, r1, r2, p1, p2);
    return;
  }

  float* part = a.partials;
  const int64_t rows = a.rows;
  if (r1 < a.rows) part[split * rows + r1] = p1;
  if (r2 < a.rows) part[split * rows + r2] = p2;
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = old == (uint32_t)(a.n_splits - 1);
    if (last)
      __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = last;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  float s1 = 0.0f, s2 = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    if (r1 < a.rows) s1 += part[s * rows + r1];
    if (r2 < a.rows) s2 += part[s * rows + r2];
  }
  epilogue<EPI>(a, r1, r2, s1, s2);
}

template <int FF, int AF, bool STAGED>
hipError_t launch_epi(const GemvArgs& a, int32_t epi, hipStream_t s) {
  const dim3 grid(a.n_tiles * a.splits_here), block(kGemvThreads);
  if (epi == kEpiGlu)
    hipLaunchKernelGGL((gemv_kernel<FF, AF, STAGED, kEpiGlu>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<FF, AF, STAGED, kEpiPlain>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int FF, int AF>
hipError_t launch_staged(const GemvArgs& a, bool staged, int32_t epi, hipStream_t s) {
  return staged ? launch_epi<FF, AF, true>(a, epi, s) : launch_epi<FF, AF, false>(a, epi, s);
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, int32_t full_fmt, int32_t approx_fmt, bool staged,
                       int32_t epi, hipStream_t s) {
  if (full_fmt == kFp16) {
    if (approx_fmt == kNone) return launch_staged<kFp16, kNone>(a, staged, epi, s);
    if (approx_fmt == kInt4) return launch_staged<kFp16, kInt4>(a, staged, epi, s);
    if (approx_fmt == kInt2) return launch_staged<kFp16, kInt2>(a, staged, epi, s);
  } else if (full_fmt == kInt4) {
    if (approx_fmt == kNone) return launch_staged<kInt4, kNone>(a, staged, epi, s);
    if (approx_fmt == kInt4) return launch_staged<kInt4, kInt4>(a, staged, epi, s);
    if (approx_fmt == kInt2) return launch_staged<kInt4, kInt2>(a, staged, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spax
