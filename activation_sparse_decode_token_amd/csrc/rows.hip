// Row-sliced tiered product with fused tier selection (gfx950).
//
// SpAx page, section 2 Eq. 1 and section 5, Figure 2 steps 3-5:
//   y = sum_{j in F} x_j W[:, j] + sum_{j in A} x_j W^[:, j]
// Every workgroup ranks x itself (the same selection as the stand-alone plan
// kernel) and then computes whole output rows -- every selected column --
// for its rows. No partial sum leaves the workgroup, so there is no
// cross-workgroup reduction and no fixed cost for one at the end of the
// launch; the price is that every workgroup walks the whole list, with small
// per-column segments. The host picks this kernel where a split-column
// product would need many splits per row tile (few rows, as in the 4096-row
// attention projections).
//
// Work decomposition
//   * Chunks of 16 stored rows. Workgroup b takes chunks c, c + G, c + 2G, ...
//     (G workgroups, at most M chunks each; G * M covers all chunks), where
//     c = xcd_order(b) gives the G / 8 workgroups that run on one XCD
//     (blocks are dealt to the 8 XCDs round-robin) consecutive chunks: the
//     chunks that share a cache line (4 for fp16, 16 for int4) then share
//     that XCD's L2 and the line crosses the fabric once. With
//     the GLU-interleaved layout a chunk is 16 gate rows and the matching 16
//     up rows, so the workgroup forms a = silu(g) * u itself.
//     A chunk never straddles a 128-row group: a code column has one scale
//     per chunk.
//   * The workgroup's list (full tier, then approx tier) is in LDS. Its 8
//     waves take contiguous eighths of each tier. Lane l serves list slot
//     l >> 1 of the wave's current 32-column round and rows 8 * (l & 1) ..
//     8 * (l & 1) + 7 of each chunk: one 16-byte (fp16), 4-byte (int4) or
//     2-byte (int2) load per chunk, addressed per lane through the tier's
//     buffer resource.
//   * Rounds are batched and double-buffered: the loads of the next batch
//     are issued before the current one is consumed. Slots past the end of
//     the list reload the last column and add it times zero.
//   * Code columns: x_j * s_{j,g} is formed per chunk when the batch is
//     consumed, the unsigned code is accumulated and the code offset removed
//     once through a running sum (as in the split-column kernel).
//   * Reduction: DPP adds over the 8 lanes of a 16-lane row that serve the
//     same row half, then a fixed-order sum over the 4 rows and 8 waves in
//     LDS. Results are bitwise reproducible.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "block_common.h"
#include "spax_internal.h"

namespace spax {
namespace {

// v + the value of the lane selected by DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 8 lanes of this lane's 16-lane row with the same lane bit 0:
// rotate by 8, by 4 (row_ror), then swap lane pairs (quad_perm 2,3,0,1).
__device__ __forceinline__ float row_half_sum(float v) {
  v = dpp_add<0x128>(v);
  v = dpp_add<0x124>(v);
  v = dpp_add<0x4E>(v);
  return v;
}

// Stream list positions [p_lo, p_hi) of one tier for the P chunks of this
// lane (rowoff[p] = first stored row of the lane's 8 rows in chunk p).
template <int FMT, int P>
__device__ __forceinline__ void rows_tier(float (&acc)[P][8], float (&corr)[P],
                                          const uint8_t* base, int64_t stride, uint32_t bytes,
                                          const uint16_t* __restrict__ scales, int64_t sstride,
                                          const int32_t* lidx, const float* lx, int p_lo,
                                          int p_hi, const int (&rowoff)[P], int lane) {
  using T = Tier<FMT>;
  constexpr bool kCode = FMT != kFp16;
  // rounds per batch: about 8 fp16 or 16 code loads per batch and lane
  constexpr int U = kCode ? (P >= 16 ? 1 : 16 / P) : (P >= 8 ? 1 : 8 / P);
  if (p_lo >= p_hi) return;
  const __amdgpu_buffer_rsrc_t rs = tier_rsrc(base, bytes);
  const uint32_t cstride = (uint32_t)stride;
  uint32_t off[P];
  int grp[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    off[p] = T::offset(rowoff[p], 0);
    grp[p] = rowoff[p] >> 7;
  }
  const int slot = lane >> 1;
  const int last = p_hi - 1;
  struct Batch {
    typename T::V v[U][P];
    uint32_t s[U][P];  // raw fp16 scales (code tiers)
    float x[U];
  };
  auto issue = [&](int q0, Batch& b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + 32 * u + slot;
      const int qc = min(q, last);
      const uint32_t col = (uint32_t)lidx[qc];
      b.x[u] = q <= last ? lx[qc] : 0.0f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        b.v[u][p] = T::load(rs, off[p] + col * cstride, 0u);
        if constexpr (kCode) b.s[u][p] = scales[(int64_t)col * sstride + grp[p]];
      }
    }
  };
  auto use = [&](const Batch& b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float f = kCode ? b.x[u] * h2f(b.s[u][p]) : b.x[u];
        T::fma(acc[p], corr[p], b.v[u][p], f);
      }
    }
  };
  constexpr int kStep = 32 * U;
  Batch b0, b1;
  int q = p_lo;
  issue(q, b0);
  for (;;) {
    if (q + kStep < p_hi) {
      issue(q + kStep, b1);
      use(b0);
    } else {
      use(b0);
      break;
    }
    q += kStep;
    if (q + kStep < p_hi) {
      issue(q + kStep, b0);
      use(b1);
    } else {
      use(b1);
      break;
    }
    q += kStep;
  }
}

// Workgroup b -> first chunk: workgroups b = 8 i + x (x = XCD) of the first
// 8 * floor(G / 8) take consecutive chunks x * floor(G / 8) + i; the rest
// keep their index. A bijection on [0, G).
__device__ __forceinline__ int xcd_order(int b, int g) {
  const int per = g >> 3;
  if (b >= 8 * per) return b;
  return (b & 7) * per + (b >> 3);
}

template <int AF, int EPI, int M, int E>
__global__ __launch_bounds__(kGemvThreads) void rows_kernel(GemvArgs a) {
  constexpr int P = EPI == kEpiGlu ? 2 * M : M;  // 16-row chunk parts
  // the rank scratch is dead once the list is in LDS; the wave sums reuse it
  union Scratch {
    RankShared rank;
    float red[kWaves][4][P][16];
  };
  __shared__ Scratch sm;
  __shared__ int32_t lidx[kRowListCap];
  __shared__ float lx[kRowListCap];
  __shared__ float fin[EPI == kEpiGlu ? P : 1][16];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int b = xcd_order(blockIdx.x, a.grid);
  // chunk m of this workgroup (a missing last chunk repeats chunk b; its
  // rows are computed and not stored)
  auto chunk = [&](int m) { return b + a.grid * m; };
  auto part_row = [&](int p) {  // first stored row of part p
    const int m = EPI == kEpiGlu ? p >> 1 : p;
    const int c = chunk(m) < a.n_chunks ? chunk(m) : b;
    if constexpr (EPI == kEpiGlu) return 256 * (c >> 3) + kChunkRows * (c & 7) + 128 * (p & 1);
    return kChunkRows * c;
  };

  rank_piece<E>(a, sm.rank, lidx, lx, 0, a.k_full, 0, a.k_approx, blockIdx.x == 0);

  float acc[P][8];
  float corr[P];
  int rowoff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    corr[p] = 0.0f;
    rowoff[p] = part_row(p) + 8 * (lane & 1);
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[p][r] = 0.0f;
  }
  const int kf = a.k_full, ka = a.k_approx;
  rows_tier<kFp16, P>(acc, corr, a.full_base, a.full_stride, a.full_bytes, nullptr, 0, lidx, lx,
                      (kf * wave) / kWaves, (kf * (wave + 1)) / kWaves, rowoff, lane);
  if constexpr (AF != kNone) {
    rows_tier<AF, P>(acc, corr, a.approx_base, a.approx_stride, a.approx_bytes, a.approx_scales,
                     a.approx_sstride, lidx + kf, lx + kf, (ka * wave) / kWaves,
                     (ka * (wave + 1)) / kWaves, rowoff, lane);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[p][r] -= corr[p];
  }

#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[p][r] = row_half_sum(acc[p][r]);
  // lanes 0/1 of each 16-lane row hold that row's sums for row halves 0/1
  if ((lane & 14) == 0) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float4* dst = reinterpret_cast<float4*>(&sm.red[wave][lane >> 4][p][8 * (lane & 1)]);
      dst[0] = make_float4(acc[p][0], acc[p][1], acc[p][2], acc[p][3]);
      dst[1] = make_float4(acc[p][4], acc[p][5], acc[p][6], acc[p][7]);
    }
  }
  __syncthreads();
  if (t < P * kChunkRows) {
    const int p = t >> 4, i = t & 15;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int g = 0; g < 4; ++g) s += sm.red[w][g][p][i];
    if constexpr (EPI == kEpiPlain) {
      if (chunk(p) < a.n_chunks) a.y[part_row(p) + i] = f2h(s);
    } else {
      fin[p][i] = s;
    }
  }
  if constexpr (EPI == kEpiGlu) {
    __syncthreads();
    if (t < M * kChunkRows) {
      const int m = t >> 4, i = t & 15;
      if (chunk(m) < a.n_chunks) store_glu(a, part_row(2 * m) + i, fin[2 * m][i], fin[2 * m + 1][i]);
    }
  }
}

template <int AF, int EPI, int M>
hipError_t launch_m(const GemvArgs& a, hipStream_t s) {
  const dim3 grid(a.grid), block(kGemvThreads);
  if (a.n <= kGemvThreads * 8)
    hipLaunchKernelGGL((rows_kernel<AF, EPI, M, 8>), grid, block, 0, s, a);
  else if (a.n <= kGemvThreads * 16)
    hipLaunchKernelGGL((rows_kernel<AF, EPI, M, 16>), grid, block, 0, s, a);
  else if (a.n <= kGemvThreads * 32)
    hipLaunchKernelGGL((rows_kernel<AF, EPI, M, 32>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int AF, int EPI>
hipError_t launch_epi(const GemvArgs& a, int32_t m, hipStream_t s) {
  if (m == 1) return launch_m<AF, EPI, 1>(a, s);
  if (m == 2) return launch_m<AF, EPI, 2>(a, s);
  if (m == 3) return launch_m<AF, EPI, 3>(a, s);
  return hipErrorInvalidValue;
}

template <int AF>
hipError_t launch_af(const GemvArgs& a, int32_t epi, int32_t m, hipStream_t s) {
  if (epi == kEpiGlu) return launch_epi<AF, kEpiGlu>(a, m, s);
  return launch_epi<AF, kEpiPlain>(a, m, s);
}

}  // namespace

hipError_t launch_rows(const GemvArgs& a, int32_t approx_fmt, int32_t epi, int32_t m,
                       hipStream_t s) {
  if (approx_fmt == kNone) return launch_af<kNone>(a, epi, m, s);
  if (approx_fmt == kInt4) return launch_af<kInt4>(a, epi, m, s);
  if (approx_fmt == kInt2) return launch_af<kInt2>(a, epi, m, s);
  return hipErrorInvalidValue;
}

}  // namespace spax
