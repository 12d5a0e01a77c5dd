// Tier selection spread over workgroups, for long inputs (gfx950).
//
// SpAx page, section 2 (magnitude top-k) and section 5, Figure 2 step 3 with
// section 5.2: the k_full largest |x_j| go to the full tier, the next
// k_approx to the approx tier; equal magnitudes rank the lower index first;
// the lists come out ascending. Same selection as the in-workgroup rank of
// the product kernel and the one-workgroup plan kernel.
//
// The input is cut into slices of 4096 entries, one 1024-thread workgroup
// each (4 entries per thread), and the two-level radix select runs as four
// short launches that meet through a small workspace region:
//   1. per-slice 256-bin histograms of key bits 14..7;
//   2. every workgroup adds the slice histograms, finds the bins holding rank
//      k_full and k_full + k_approx, and writes per-slice 128-bin histograms
//      of the entries inside those two bins;
//   3. every workgroup adds those, finds the boundary keys t1, t2 and the tie
//      quotas q1, q2, and writes its slice's counts of (key > t1, key == t1,
//      key > t2, key == t2);
//   4. (when the caller wants lists in memory) every workgroup adds the
//      counts of the slices before its own, scans its slice and writes its
//      entries' list positions. The fused product skips this step: its
//      workgroups place their own pieces from the slice counts.
// Each workgroup handles 4096 entries instead of every workgroup of the
// product ranking all n, which is what makes long inputs (the 11008- and
// 28672-wide down projections) expensive in the fused form.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "block_common.h"
#include "spax_internal.h"

namespace spax {
namespace {

constexpr int kSliceE = kSliceEntries / kGemvThreads;  // entries per thread
static_assert(kSliceE == 4, "slices of 4 entries per thread");

// This thread's 4 raw fp16 entries of slice s (0 past n), two per register,
// and how many are real.
__device__ __forceinline__ int load_slice(const uint16_t* __restrict__ x, int n, int s,
                                          uint32_t (&xr)[2]) {
  const int base = s * kSliceEntries + 4 * (int)threadIdx.x;
  if (base + 3 < n) {
    const uint2 v = *reinterpret_cast<const uint2*>(x + base);
    xr[0] = v.x;
    xr[1] = v.y;
  } else {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const uint32_t lo = base + j < n ? x[base + j] : 0u;
      const uint32_t hi = base + j + 1 < n ? x[base + j + 1] : 0u;
      xr[j / 2] = lo | (hi << 16);
    }
  }
  return max(0, min(4, n - base));
}

__global__ __launch_bounds__(kGemvThreads) void sel_hist_kernel(const uint16_t* __restrict__ x,
                                                                 int n, SelectScratch* ws) {
  __shared__ uint32_t hist[257];
  const int t = threadIdx.x, s = blockIdx.x;
  uint32_t xr[2];
  const int nv = load_slice(x, n, s, xr);
  if (t < 257) hist[t] = 0u;
  __syncthreads();
  hist_add<kSliceE>(hist, [&](int i) {
    return i < nv ? (int)((rawbits(xr, i) & 0x7FFFu) >> 7) : 256;
  });
  __syncthreads();
  if (t < 256) ws->hist[s][t] = hist[t];
}

__global__ __launch_bounds__(kGemvThreads) void sel_sub_kernel(const uint16_t* __restrict__ x,
                                                                int n, int k_full, int k_approx,
                                                                int slices, SelectScratch* ws) {
  __shared__ uint32_t tot[256];
  __shared__ uint32_t sub[2][128];
  __shared__ int32_t sel[4];
  const int t = threadIdx.x, s = blockIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const uint32_t K1 = (uint32_t)k_full, K2 = (uint32_t)(k_full + k_approx);
  uint32_t xr[2];
  const int nv = load_slice(x, n, s, xr);
  if (t < 256) {
    uint32_t v = 0u;
    for (int q = 0; q < slices; ++q) v += ws->hist[q][t];
    tot[t] = v;
    (&sub[0][0])[t] = 0u;
  }
  __syncthreads();
  // bins holding rank K1 and rank K2 and the entries above them (wave 0)
  if (wave == 0) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = tot[4 * lane + j];
    uint32_t above = wave_excl_suffix(c[0] + c[1] + c[2] + c[3]);
    int s1 = -1, s2 = -1;
    uint32_t x1 = 0u, x2 = 0u;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (K1 > 0 && above < K1 && K1 <= above + c[j]) { s1 = 4 * lane + j; x1 = above; }
      if (K2 > 0 && above < K2 && K2 <= above + c[j]) { s2 = 4 * lane + j; x2 = above; }
      above += c[j];
    }
    int b;
    uint32_t v;
    wave_pick(s1, x1, b, v);
    if (lane == 0) { sel[0] = b; sel[1] = (int32_t)v; }
    wave_pick(s2, x2, b, v);
    if (lane == 0) { sel[2] = b; sel[3] = (int32_t)v; }
  }
  __syncthreads();
  const int b1 = sel[0], b2 = sel[2];
  auto sub_bin = [&](int i, int b) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const int hb = i < nv ? (int)(k >> 7) : 256;
    return hb == b ? (int)(k & 127u) : -1;
  };
  hist_add<kSliceE>(sub[0], [&](int i) { return sub_bin(i, b1); });
  hist_add<kSliceE>(sub[1], [&](int i) { return sub_bin(i, b2); });
  __syncthreads();
  if (t < 256) (&ws->sub[s][0][0])[t] = (&sub[0][0])[t];
  if (s == 0 && t < 4) ws->sel[t] = sel[t];
}

__global__ __launch_bounds__(kGemvThreads) void sel_count_kernel(const uint16_t* __restrict__ x,
                                                                  int n, int k_full, int k_approx,
                                                                  int slices, SelectScratch* ws) {
  __shared__ uint32_t sub[2][128];
  __shared__ uint32_t tq[4];
  __shared__ uint32_t part[4][kWaves];
  const int t = threadIdx.x, s = blockIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const uint32_t K1 = (uint32_t)k_full, K2 = (uint32_t)(k_full + k_approx);
  uint32_t xr[2];
  const int nv = load_slice(x, n, s, xr);
  if (t < 256) {
    uint32_t v = 0u;
    for (int q = 0; q < slices; ++q) v += (&ws->sub[q][0][0])[t];
    (&sub[0][0])[t] = v;
  }
  __syncthreads();
  // boundary keys t (kAboveAll when the tier is empty) and quotas q (wave 0)
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = ws->sel[2 * r];
      const uint32_t ab = (uint32_t)ws->sel[2 * r + 1];
      const uint32_t K = r == 0 ? K1 : K2;
      int key = (int)kAboveAll;
      uint32_t quota = 0u;
      if (b >= 0) {  // wave-uniform
        const uint32_t c0 = sub[r][2 * lane], c1 = sub[r][2 * lane + 1];
        uint32_t above = ab + wave_excl_suffix(c0 + c1);
        int sk = -1;
        uint32_t sq = 0u;
        if (above < K && K <= above + c1) { sk = (b << 7) | (2 * lane + 1); sq = K - above; }
        above += c1;
        if (above < K && K <= above + c0) { sk = (b << 7) | (2 * lane); sq = K - above; }
        wave_pick(sk, sq, key, quota);
      }
      if (lane == 0) {
        tq[2 * r] = (uint32_t)key;
        tq[2 * r + 1] = quota;
      }
    }
  }
  __syncthreads();
  const uint32_t t1 = tq[0], t2 = tq[2];
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kSliceE; ++i) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool ok = i < nv;
    c[0] += ok && k > t1;
    c[1] += ok && k == t1;
    c[2] += ok && k > t2;
    c[3] += ok && k == t2;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(c[j]), 63);
    if (lane == 0) part[j][wave] = w;
  }
  __syncthreads();
  if (t < 4) {
    uint32_t v = 0u;
    for (int w = 0; w < kWaves; ++w) v += part[t][w];
    ws->cnt[s][t] = v;
    if (s == 0) ws->sel[4 + t] = (int32_t)tq[t];
  }
}

__global__ __launch_bounds__(kGemvThreads) void sel_place_kernel(
    const uint16_t* __restrict__ x, int n, SelectScratch* ws, int32_t* __restrict__ full_idx,
    int32_t* __restrict__ approx_idx) {
  __shared__ uint32_t scan[2][kWaves];
  const int t = threadIdx.x, s = blockIdx.x;
  const int lane = t & 63, wave = t >> 6;
  uint32_t xr[2];
  const int nv = load_slice(x, n, s, xr);
  const uint32_t t1 = (uint32_t)ws->sel[4], q1 = (uint32_t)ws->sel[5];
  const uint32_t t2 = (uint32_t)ws->sel[6], q2 = (uint32_t)ws->sel[7];
  // counts of the slices before this one
  uint32_t pre[4] = {0u, 0u, 0u, 0u};
  for (int q = 0; q < s; ++q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pre[j] += ws->cnt[q][j];
  }
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kSliceE; ++i) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool ok = i < nv;
    c[0] += ok && k > t1;
    c[1] += ok && k == t1;
    c[2] += ok && k > t2;
    c[3] += ok && k == t2;
  }
  // in-slice exclusive prefixes, packed two counts per register (each below
  // 2^16: at most 4096 per slice)
  const uint32_t p01 = c[0] | (c[1] << 16), p23 = c[2] | (c[3] << 16);
  const uint32_t i01 = wave_incl_scan(p01), i23 = wave_incl_scan(p23);
  if (lane == 63) {
    scan[0][wave] = i01;
    scan[1][wave] = i23;
  }
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t wt =
      (lane >> 4) < 2 && (lane & 15) < kWaves ? scan[lane >> 4][lane & 15] : 0u;
  const uint32_t wex = row16_incl_scan(wt) - wt;
  const uint32_t ex01 = (uint32_t)__builtin_amdgcn_readlane((int)wex, wv) + i01 - p01;
  const uint32_t ex23 = (uint32_t)__builtin_amdgcn_readlane((int)wex, 16 + wv) + i23 - p23;
  uint32_t g1 = pre[0] + (ex01 & 0xFFFFu), e1r = pre[1] + (ex01 >> 16);
  uint32_t g2 = pre[2] + (ex23 & 0xFFFFu), e2r = pre[3] + (ex23 >> 16);
  const int base = s * kSliceEntries + 4 * t;
#pragma unroll
  for (int i = 0; i < kSliceE; ++i) {
    const uint32_t k = rawbits(xr, i) & 0x7FFFu;
    const bool ok = i < nv;
    const bool gt1 = ok && k > t1, eq1 = ok && k == t1;
    const bool gt2 = ok && k > t2, eq2 = ok && k == t2;
    const bool in_f = gt1 || (eq1 && e1r < q1);
    const bool in_fa = gt2 || (eq2 && e2r < q2);
    const uint32_t fpos = g1 + min(e1r, q1);          // F entries before this one
    const uint32_t apos = g2 + min(e2r, q2) - fpos;   // A entries before this one
    if (in_f) full_idx[fpos] = base + i;
    else if (in_fa) approx_idx[apos] = base + i;
    g1 += gt1;
    e1r += eq1;
    g2 += gt2;
    e2r += eq2;
  }
}

}  // namespace

hipError_t launch_select(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                         int32_t* full_idx, int32_t* approx_idx, SelectScratch* ws,
                         hipStream_t s) {
  const int slices = (n + kSliceEntries - 1) / kSliceEntries;
  if (n < 1 || slices > kMaxSlices) return hipErrorInvalidValue;
  const dim3 grid(slices), block(kGemvThreads);
  hipLaunchKernelGGL(sel_hist_kernel, grid, block, 0, s, x, n, ws);
  hipLaunchKernelGGL(sel_sub_kernel, grid, block, 0, s, x, n, k_full, k_approx, slices, ws);
  hipLaunchKernelGGL(sel_count_kernel, grid, block, 0, s, x, n, k_full, k_approx, slices, ws);
  if (full_idx)
    hipLaunchKernelGGL(sel_place_kernel, grid, block, 0, s, x, n, ws, full_idx, approx_idx);
  return hipGetLastError();
}

}  // namespace spax
