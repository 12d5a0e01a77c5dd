// Tier selection for one activation vector (gfx950).
//
// SpAx page, section 2 (magnitude top-k) and section 5, Figure 2 step 3 with
// section 5.2: rank the entries of x by |x_j|; the k_full largest go to the
// full tier, the next k_approx to the middle tier, the rest are skipped.
// Equal magnitudes rank the lower index first; lists come out ascending.
//
// One workgroup of 1024 threads. Thread t owns the E consecutive entries
// [t*E, t*E+E), keeping their 15-bit magnitude keys in registers.
//   1. 256-bin histogram of key bits 14..7 (per-wave LDS histograms).
//   2. Suffix counts locate the bins holding rank k_full and rank
//      k_full + k_approx (counted from the largest).
//   3. 128-bin histograms of bits 6..0 inside those two bins give the exact
//      boundary keys t1, t2 and how many entries equal to each boundary key
//      are kept (q1, q2).
//   4. A block scan of "key == t" counts in index order gives every entry its
//      rank among equal keys, which decides the boundary ties; a second block
//      scan of tier counts gives the output positions (ascending by index).
#include <hip/hip_runtime.h>

#include "spax_internal.h"

namespace spax {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr uint32_t kNoKey = 0xFFFFu;     // padding beyond n
constexpr uint32_t kAboveAll = 0x8000u;  // boundary key when a tier is empty

__device__ __forceinline__ void wave_incl_scan2(uint32_t& a, uint32_t& b, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t ta = __shfl_up(a, d, 64);
    const uint32_t tb = __shfl_up(b, d, 64);
    if (lane >= d) {
      a += ta;
      b += tb;
    }
  }
}

// Exclusive scan of (a, b) over the block in thread order.
__device__ __forceinline__ void block_excl_scan2(uint32_t& a, uint32_t& b, uint32_t* sm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t ia = a, ib = b;
  wave_incl_scan2(ia, ib, lane);
  if (lane == 63) {
    sm[wave] = ia;
    sm[kPlanWaves + wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  for (int w = 0; w < wave; ++w) {
    pa += sm[w];
    pb += sm[kPlanWaves + w];
  }
  __syncthreads();
  a = pa + ia - a;
  b = pb + ib - b;
}

// Suffix sum over the 64 lanes: returns sum of v over lanes > lane.
__device__ __forceinline__ uint32_t wave_excl_suffix(uint32_t v, int lane) {
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_down(incl, d, 64);
    if (lane + d < 64) incl += t;
  }
  return incl - v;
}

template <int E>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const uint16_t* __restrict__ x, int n, int k_full, int k_approx,
    int32_t* __restrict__ full_idx, int32_t* __restrict__ approx_idx) {
  __shared__ uint32_t hist[kPlanWaves][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t sub[2][128];
  __shared__ uint32_t scan_sm[2 * kPlanWaves];
  // [0] bin of rank K1, [1] count above it, [2],[3] same for K2,
  // [4] t1, [5] q1, [6] t2, [7] q2
  __shared__ int32_t sel[8];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int base = t * E;
  const uint32_t K1 = (uint32_t)k_full;
  const uint32_t K2 = (uint32_t)(k_full + k_approx);

  uint32_t key[E];
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    if (base + i + 3 < n) {
      const uint2 v = *reinterpret_cast<const uint2*>(x + base + i);
      key[i + 0] = v.x & 0x7FFFu;
      key[i + 1] = (v.x >> 16) & 0x7FFFu;
      key[i + 2] = v.y & 0x7FFFu;
      key[i + 3] = (v.y >> 16) & 0x7FFFu;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        key[i + j] = (base + i + j < n) ? (uint32_t)(x[base + i + j] & 0x7FFFu) : kNoKey;
    }
  }

  for (int i = t; i < kPlanWaves * 256; i += kPlanThreads) (&hist[0][0])[i] = 0;
  if (t < 256) (&sub[0][0])[t] = 0;
  if (t == 0) {
    sel[0] = -1; sel[1] = 0; sel[2] = -1; sel[3] = 0;
    sel[4] = (int32_t)kAboveAll; sel[5] = 0; sel[6] = (int32_t)kAboveAll; sel[7] = 0;
  }
  __syncthreads();

  // 1. top-level histogram
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (key[i] != kNoKey) atomicAdd(&hist[wave][key[i] >> 7], 1u);
  __syncthreads();
  if (t < 256) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) s += hist[w][t];
    tot[t] = s;
  }
  __syncthreads();

  // 2. bins holding rank K1 and rank K2 (1-based, from the largest key)
  if (wave == 0) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = tot[4 * lane + j];
    uint32_t above = wave_excl_suffix(c[0] + c[1] + c[2] + c[3], lane);
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (K1 > 0 && above < K1 && K1 <= above + c[j]) { sel[0] = 4 * lane + j; sel[1] = (int32_t)above; }
      if (K2 > 0 && above < K2 && K2 <= above + c[j]) { sel[2] = 4 * lane + j; sel[3] = (int32_t)above; }
      above += c[j];
    }
  }
  __syncthreads();

  // 3. low-level histograms inside the two boundary bins
  const int b1 = sel[0];
  const int b2 = sel[2];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (key[i] == kNoKey) continue;
    const int hb = (int)(key[i] >> 7);
    if (hb == b1) atomicAdd(&sub[0][key[i] & 127u], 1u);
    if (hb == b2) atomicAdd(&sub[1][key[i] & 127u], 1u);
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = r == 0 ? b1 : b2;
      const uint32_t K = r == 0 ? K1 : K2;
      if (b < 0) continue;
      const uint32_t c0 = sub[r][2 * lane], c1 = sub[r][2 * lane + 1];
      uint32_t above = (uint32_t)sel[1 + 2 * r] + wave_excl_suffix(c0 + c1, lane);
      if (above < K && K <= above + c1) {
        sel[4 + 2 * r] = (b << 7) | (2 * lane + 1);
        sel[5 + 2 * r] = (int32_t)(K - above);
      }
      above += c1;
      if (above < K && K <= above + c0) {
        sel[4 + 2 * r] = (b << 7) | (2 * lane);
        sel[5 + 2 * r] = (int32_t)(K - above);
      }
    }
  }
  __syncthreads();

  // 4. ranks among equal boundary keys, tiers, output positions
  const uint32_t t1 = (uint32_t)sel[4], q1 = (uint32_t)sel[5];
  const uint32_t t2 = (uint32_t)sel[6], q2 = (uint32_t)sel[7];
  uint32_t r1 = 0, r2 = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    r1 += key[i] == t1;
    r2 += key[i] == t2;
  }
  block_excl_scan2(r1, r2, scan_sm);

  uint32_t nf = 0, na = 0;
  {
    uint32_t e1 = r1, e2 = r2;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t k = key[i];
      if (k == kNoKey) continue;
      const bool in_f = k > t1 || (k == t1 && e1 < q1);
      const bool in_fa = k > t2 || (k == t2 && e2 < q2);
      e1 += k == t1;
      e2 += k == t2;
      nf += in_f;
      na += (!in_f && in_fa);
    }
  }
  uint32_t of = nf, oa = na;
  block_excl_scan2(of, oa, scan_sm);
  {
    uint32_t e1 = r1, e2 = r2;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t k = key[i];
      if (k == kNoKey) continue;
      const bool in_f = k > t1 || (k == t1 && e1 < q1);
      const bool in_fa = k > t2 || (k == t2 && e2 < q2);
      e1 += k == t1;
      e2 += k == t2;
      // the counts are exact by construction; the bounds only keep a logic
      // error from writing past a caller's list
      if (in_f) {
        if (of < K1) full_idx[of] = base + i;
        ++of;
      } else if (in_fa) {
        if (oa < (uint32_t)k_approx) approx_idx[oa] = base + i;
        ++oa;
      }
    }
  }
}

}  // namespace

hipError_t launch_plan(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                       int32_t* full_idx, int32_t* approx_idx, hipStream_t s) {
  const dim3 grid(1), block(kPlanThreads);
  if (n <= kPlanThreads * 4)
    hipLaunchKernelGGL(plan_kernel<4>, grid, block, 0, s, x, n, k_full, k_approx, full_idx, approx_idx);
  else if (n <= kPlanThreads * 8)
    hipLaunchKernelGGL(plan_kernel<8>, grid, block, 0, s, x, n, k_full, k_approx, full_idx, approx_idx);
  else if (n <= kPlanThreads * 16)
    hipLaunchKernelGGL(plan_kernel<16>, grid, block, 0, s, x, n, k_full, k_approx, full_idx, approx_idx);
  else if (n <= kPlanThreads * 32)
    hipLaunchKernelGGL(plan_kernel<32>, grid, block, 0, s, x, n, k_full, k_approx, full_idx, approx_idx);
  else
    hipLaunchKernelGGL(plan_kernel<64>, grid, block, 0, s, x, n, k_full, k_approx, full_idx, approx_idx);
  return hipGetLastError();
}

}  // namespace spax
