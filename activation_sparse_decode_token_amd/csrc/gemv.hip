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
//   * Every split takes the same share of each tier's list (F positions
//     [k_f s / S, k_f (s+1) / S) and the same share of A), so every
//     workgroup gets the same mix of bytes and dequantisation work.
//     Workgroup (split, tile) streams its piece for its tile; its 16 waves
//     take contiguous sixteenths of each tier's piece.
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
//   * Group-128 code tiers fold 2^b x_j s_{j,g} into one fp32 factor per
//     column and lane, turn each code u into the fp16 value 1 + u / 2^b with
//     bit operations and multiply it in with fp16 x fp32 FMAs; the constant
//     part (2^b plus the code offset, 8 for int4, 1.5 for int2) is removed
//     once at the end through a per-lane running sum. The two-scale sign
//     code adds +-x_j s_{j,0} +-x_j s_{j,1} per weight (signs moved into fp16
//     1.0s); the trellis code looks each weight's 16-bit window up in a
//     codebook held in LDS (section 5.1 of the SpAx page).
//   * The 16 wave partials are added in LDS in a fixed order (in two halves
//     for the trellis kernels, whose codebook takes 128 KB of LDS). With one split
//     the workgroup writes y; otherwise each workgroup stores its fp32 partial
//     and the last workgroup of a tile (agent-scope counter) adds the n_splits
//     partials in split order and writes y (arrivals are counted in two
//     levels, groups of 8 splits, to keep contention on one counter low).
//     Counters are reset by the workgroups that complete them. The
//     summation order never depends on timing, so results are bitwise
//     reproducible.
//   * The tiles of one split run on one XCD (blocks are dealt to the 8 XCDs
//     round-robin), so the shared lines of a split hit that XCD's L2.
//   * Gate/up epilogue: with the GLU-interleaved layout a tile holds 256 gate
//     rows and the matching 256 up rows, so the final reduction forms
//     a = silu(g) * u (SpAx page, section 2) from the fp16-rounded g and u.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "block_common.h"
#include "stream_common.h"
#include "spax_internal.h"

namespace spax {
namespace {

// Block -> (split, tile): groups of 8 consecutive splits are interleaved so
// that block b and split (b mod 8) coincide on the XCD that runs block b.
// (unsigned 32-bit arithmetic: the divisions are short on the scalar unit)
__device__ __forceinline__ void map_block(uint32_t b, uint32_t n_tiles, uint32_t splits_here,
                                          int& s_loc, int& tile) {
  const uint32_t groups = splits_here >> 3;
  const uint32_t fb = groups * 8u * n_tiles;
  if (b < fb) {
    const uint32_t g = b / (8u * n_tiles);
    const uint32_t r = b - g * 8u * n_tiles;
    s_loc = (int)(g * 8u + (r & 7u));
    tile = (int)(r >> 3);
  } else {
    const uint32_t r = b - fb;
    const uint32_t q = r / n_tiles;
    s_loc = (int)(groups * 8u + q);
    tile = (int)(r - q * n_tiles);
  }
}

template <int FF, int AF, int MODE, int EPI, int E>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  // The rank scratch is dead once the list piece is in LDS; the wave
  // partials reuse it.
  // The trellis tier keeps its 128 KB codebook in LDS; its kernels then add
  // the 16 wave partials in two halves and have no code-factor rows.
  constexpr bool kTrel = AF == kTrellis;
  constexpr int kRedWaves = kTrel ? kWaves / 2 : kWaves;
  union Scratch {
    RankShared rank;
    float red[kRedWaves][kTileRows];
  };
  __shared__ Scratch sm;
  constexpr bool kPiece = MODE == kListRank || MODE == kListSliced;  // list piece in LDS
  constexpr int kCap = kTrel ? kListCapTrellis : kListCap;
  __shared__ int32_t lidx[kPiece ? kCap : 1];
  __shared__ float lx[kPiece ? kCap : 1];
  __shared__ WaveMeta wmeta[kTrel ? 1 : 2][kTrel ? 1 : kWaves];  // per tier and wave
  __shared__ __attribute__((aligned(16))) uint16_t cbk[kTrel ? 65536 : 8];
  __shared__ uint32_t last_flag;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if constexpr (kTrel) {
    // the codebook into LDS (8192 16-byte pieces, 8 per thread) first: with
    // the fused ranking its latency overlaps the ranking; it is complete
    // after the barrier below
    const uint4* src = reinterpret_cast<const uint4*>(a.codebook);
    uint4* dst = reinterpret_cast<uint4*>(cbk);
#pragma unroll
    for (int k = 0; k < 65536 / 8 / kGemvThreads; ++k)
      dst[t + k * kGemvThreads] = src[t + k * kGemvThreads];
  }
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
  if constexpr (kPiece) {
    // the piece holds F positions [f0, f1) then A positions [a0, a1)
    if constexpr (MODE == kListRank)
      rank_piece<E>(a, sm.rank, lidx, lx, f0, f1, a0, a1, tile == 0);
    else
      place_sliced(a, sm.rank.scan, lidx, lx, f0, f1, a0, a1, tile == 0);
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
  if constexpr (kTrel) __syncthreads();  // the codebook is in LDS
  {
    const int lf = f_hi - f_lo, la = a_hi - a_lo;
    TierStream<FF, MODE> sf(wmeta[0][kTrel ? 0 : wave], a.full_base, a.full_stride,
                            a.full_bytes,
                            a.full_scales, a.full_sstride, a.full_idx, a.x, lidx, lx,
                            f_lo + (lf * wave) / kWaves, f_lo + (lf * (wave + 1)) / kWaves, row0,
                            a.rows, lane, ld_lane);
    sf.begin();
    if constexpr (AF != kNone) {
      TierStream<AF, MODE> sa(wmeta[kTrel ? 0 : 1][kTrel ? 0 : wave], a.approx_base,
                              a.approx_stride, a.approx_bytes,
                              a.approx_scales, a.approx_sstride, a.approx_idx, a.x,
                              lidx, lx, a_lo + (la * wave) / kWaves,
                              a_lo + (la * (wave + 1)) / kWaves, row0, a.rows, lane, ld_lane,
                              a.approx_seg);
      if constexpr (kTrel) sa.cbk = cbk;
      sa.begin();
      sf.run(acc, corr);
      sa.run(acc, corr);
    } else {
      sf.run(acc, corr);
    }
  }
  if constexpr (FF == kInt4 || AF != kNone) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] -= corr;
  }

  if constexpr (kTrel) {
    // waves 8..15 store, waves 0..7 add theirs: slot w holds waves w, w + 8
    float4* dst = reinterpret_cast<float4*>(&sm.red[wave & (kRedWaves - 1)][8 * lane]);
    if (wave >= kRedWaves) {
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wave < kRedWaves) {
      const float4 u0 = dst[0], u1 = dst[1];
      dst[0] = make_float4(acc[0] + u0.x, acc[1] + u0.y, acc[2] + u0.z, acc[3] + u0.w);
      dst[1] = make_float4(acc[4] + u1.x, acc[5] + u1.y, acc[6] + u1.z, acc[7] + u1.w);
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(&sm.red[wave][8 * lane]);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();

  // thread t < kTileRows owns row t of the tile from here on
  const bool owner = t < kTileRows;
  float p = 0.0f;
  if (owner) {
#pragma unroll
    for (int w = 0; w < kRedWaves; ++w) p += sm.red[w][t];
  }
  const int r = row0 + t;

  if (a.n_splits > 1) {
    // Cross-split reduction without cache-wide fences. The partials are
    // written and read with agent-scope relaxed atomics, which the gfx950
    // memory model maps to L2 write-through stores and L2-coherent loads,
    // so no L2 writeback or invalidate is needed: waiting for the stores
    // to complete before the counter increment orders them for every XCD.
    float* part = a.partials;
    const int64_t rows = a.rows;
    if (owner && r < a.rows)
      __hip_atomic_store(&part[split * rows + r], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this lane's stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (t == 0) {
      // Two-level arrival count, so that at most 8 workgroups meet on one
      // counter: the last of each group of 8 splits counts its group in,
      // the last group's last workgroup reduces (with 8 splits or fewer the
      // group's last workgroup reduces directly). Each counter is reset by
      // the workgroup that completes it.
      uint32_t* c = a.counters + tile * kCountersPerTile;
      const int g = split >> 3;
      const uint32_t gsize = (uint32_t)min(8, a.n_splits - 8 * g);
      const uint32_t ngroups = (uint32_t)((a.n_splits + 7) >> 3);
      uint32_t last = 0u;
      const uint32_t old =
          __hip_atomic_fetch_add(&c[1 + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == gsize - 1) {
        __hip_atomic_store(&c[1 + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (ngroups == 1) {  // one group: its last workgroup is the last
          last = 1u;
        } else {
          const uint32_t old2 =
              __hip_atomic_fetch_add(&c[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (old2 == ngroups - 1) {
            __hip_atomic_store(&c[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = 1u;
          }
        }
      }
      last_flag = last;
    }
    __syncthreads();
    if (!last_flag) return;
    // partials are added in split order; the loads of up to 32 splits are
    // issued together (clamped to valid addresses, unused ones not added)
    p = 0.0f;
    if (owner) {
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
  }

  if constexpr (EPI == kEpiPlain) {
    if (owner && r < a.rows) a.y[r] = f2h(p);
  } else {
    __syncthreads();
    if (owner) sm.red[0][t] = p;
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
  if (mode == kListSliced) return launch_epi<FF, AF, kListSliced, 0>(a, epi, s);
  // entries per ranking thread: the smallest of 8, 16, 24, 32, 48, 56, 64
  // that covers n (56: the 70B down projection's 28672 exactly)
  static_assert(kRankMaxN == kRankThreads * 64, "fused ranking at up to 64 entries per thread");
  if (a.n <= kRankThreads * 8) return launch_epi<FF, AF, kListRank, 8>(a, epi, s);
  if (a.n <= kRankThreads * 16) return launch_epi<FF, AF, kListRank, 16>(a, epi, s);
  if (a.n <= kRankThreads * 24) return launch_epi<FF, AF, kListRank, 24>(a, epi, s);
  if (a.n <= kRankThreads * 32) return launch_epi<FF, AF, kListRank, 32>(a, epi, s);
  if (a.n <= kRankThreads * 48) return launch_epi<FF, AF, kListRank, 48>(a, epi, s);
  if (a.n <= kRankThreads * 56) return launch_epi<FF, AF, kListRank, 56>(a, epi, s);
  if (a.n <= kRankThreads * 64) return launch_epi<FF, AF, kListRank, 64>(a, epi, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, int32_t full_fmt, int32_t approx_fmt, int32_t mode,
                       int32_t epi, hipStream_t s) {
  if (full_fmt == kFp16) {
    if (approx_fmt == kNone) return launch_mode<kFp16, kNone>(a, mode, epi, s);
    if (approx_fmt == kInt4) return launch_mode<kFp16, kInt4>(a, mode, epi, s);
    if (approx_fmt == kInt2) return launch_mode<kFp16, kInt2>(a, mode, epi, s);
    if (approx_fmt == kSign2) return launch_mode<kFp16, kSign2>(a, mode, epi, s);
    if (approx_fmt == kTrellis) return launch_mode<kFp16, kTrellis>(a, mode, epi, s);
  } else if (full_fmt == kInt4) {
    if (approx_fmt == kNone) return launch_mode<kInt4, kNone>(a, mode, epi, s);
    if (approx_fmt == kInt4) return launch_mode<kInt4, kInt4>(a, mode, epi, s);
    if (approx_fmt == kInt2) return launch_mode<kInt4, kInt2>(a, mode, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spax
