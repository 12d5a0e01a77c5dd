// Selected-column copy, packer and workspace clear (gfx950).
#include <hip/hip_fp16.h>
#include <algorithm>
#include <hip/hip_runtime.h>

#include "spax_internal.h"

namespace spax {
namespace {

// ---------------------------------------------------------------------------
// Selected-column copy for host-resident weights.
// SpAx page, section 5 Figure 2 step 4 (only the top-tier columns and the
// middle-tier codes of the selected entries are fetched into GPU memory) and
// section 5.3 (each entry's data is a contiguous range; ranges of one tier
// are read as whole runs). Each wave moves whole columns from pinned host
// memory (device-addressable) into device staging, slot = list position, so
// the product reads the staging in list order. Adjacent columns of a run
// stream back to back from the same wave-wide loads, so no per-range request
// is issued by the host.
// ---------------------------------------------------------------------------
constexpr int kCopyThreads = 256;

__device__ __forceinline__ void copy_bytes(uint8_t* __restrict__ dst,
                                           const uint8_t* __restrict__ src, int64_t nbytes,
                                           int lane) {
  // nbytes is a multiple of 16; 8 loads in flight per lane
  const int64_t n16 = nbytes >> 4;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  int64_t i = lane;
  for (; i + 7 * 64 < n16; i += 8 * 64) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s[i + u * 64];
#pragma unroll
    for (int u = 0; u < 8; ++u) d[i + u * 64] = v[u];
  }
  for (; i < n16; i += 64) d[i] = s[i];
}

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(CopyArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * (kCopyThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kCopyThreads / 64);
  const int64_t nf = a.f_hi - a.f_lo;
  const int64_t total = nf + (a.a_hi - a.a_lo);
  for (int64_t e = gw; e < total; e += nw) {
    if (e < nf) {
      const int64_t p = a.f_lo + e;
      const int64_t col = a.full_idx[p];
      copy_bytes(a.full_dst + p * a.full_bytes, a.full_src + col * a.full_bytes, a.full_bytes,
                 lane);
      for (int i = lane; i < a.fscale_n; i += 64)
        a.fscale_dst[p * a.fscale_n + i] = a.fscale_src[col * a.fscale_n + i];
    } else {
      const int64_t p = a.a_lo + (e - nf);
      const int64_t col = a.approx_idx[p];
      copy_bytes(a.approx_dst + p * a.approx_bytes, a.approx_src + col * a.approx_bytes,
                 a.approx_bytes, lane);
      for (int i = lane; i < a.ascale_n; i += 64)
        a.ascale_dst[p * a.ascale_n + i] = a.ascale_src[col * a.ascale_n + i];
    }
  }
}

// ---------------------------------------------------------------------------
// Group-128 packer (offline). SpAx page section 5, Figure 2 step 1 and
// section 5.1: every column is encoded on its own, in groups of 128 rows with
// one fp16 scale.
//   int4: s = fp16(m / 7),   q = clamp(rne(w / s), -8, 7)
//   int2: s = fp16(m / 1.5), u = clamp(rne(w / s + 1.5), 0, 3)
// The quotients are taken in fp64 and rounded once (to fp16 through fp32, or
// to an integer with ties to even); for fp16 operands neither rounding can
// land on a tie the exact quotient does not have.
// One wave per (column, group); lane l reads rows 2l and 2l+1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, int rows,
                                                   int cols, int fmt, uint8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int groups = rows / kGroup;
  if (item >= (int64_t)cols * groups) return;
  const int64_t col = item / groups;
  const int g = (int)(item - col * groups);
  const uint16_t* src = w + col * rows + (int64_t)g * kGroup;
  const float w0 = h2f(src[2 * lane]), w1 = h2f(src[2 * lane + 1]);
  float m = fmaxf(fabsf(w0), fabsf(w1));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  const double top = fmt == kInt4 ? 7.0 : 1.5;
  const __half sh = __float2half_rn((float)((double)m / top));
  const uint16_t sbits = __half_as_ushort(sh);
  const double s = (double)__half2float(sh);
  if (lane == 0) scales[col * groups + g] = sbits;
  if (fmt == kInt4) {
    int q0 = 0, q1 = 0;
    if (s > 0.0) {
      q0 = (int)rint((double)w0 / s);
      q1 = (int)rint((double)w1 / s);
      q0 = min(7, max(-8, q0));
      q1 = min(7, max(-8, q1));
    }
    codes[col * (rows / 2) + (int64_t)g * 64 + lane] =
        (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
  } else {
    // lanes 0..31 each build one byte from rows 4l .. 4l+3
    if (lane < 32) {
      uint32_t byte = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double wv = (double)h2f(src[4 * lane + r]);
        int u = 2;
        if (s > 0.0) u = min(3, max(0, (int)rint(wv / s + 1.5)));
        byte |= (uint32_t)u << (2 * r);
      }
      codes[col * (rows / 4) + (int64_t)g * 32 + lane] = (uint8_t)byte;
    }
  }
}

// ---------------------------------------------------------------------------
// Two-scale 2-bit sign packer (offline). SpAx page section 5.1, Eq. 4: a
// weight is rebuilt as e1 s0 + e2 s1 with signs e1, e2 and two scales per
// column; the codes minimise the squared error given the scales. Scales
// (closed-form greedy fit): s0 = fp16(mean |w|), s1 = fp16(mean |w - e1 s0|)
// with e1 = +1 iff w >= 0. Every fp16 value is an exact integer in units of
// 2^-24 (below 2^40 in magnitude), so the sums and the distances are exact
// 64-bit integers; each mean is one fp64 division rounded once to fp16.
// One workgroup per column.
// ---------------------------------------------------------------------------
constexpr int kSign2Threads = 256;

// fp16 bits -> signed value in units of 2^-24 (finite inputs)
__device__ __forceinline__ int64_t h_units(uint32_t b) {
  const uint32_t e = (b >> 10) & 31u, m = b & 1023u;
  const int64_t mag = e == 0u ? (int64_t)m : (int64_t)(m | 1024u) << (e - 1u);
  return (b & 0x8000u) ? -mag : mag;
}

// Round a finite v >= 0 to fp16, ties to even, in one step from the double
// (the quantum of [2^E, 2^(E+1)) is 2^(E-10), 2^-24 below 2^-14; rint rounds
// ties to even; both scalings are exact).
__device__ __forceinline__ uint16_t f64_to_h_rne(double v) {
  if (v == 0.0) return 0;
  int e;
  (void)frexp(v, &e);  // v in [2^(e-1), 2^e)
  int E = e - 1;
  if (E < -14) return (uint16_t)rint(ldexp(v, 24));  // 1024 is the smallest normal
  uint32_t q = (uint32_t)rint(ldexp(v, 10 - E));      // in [1024, 2048]
  if (q == 2048u) {
    q = 1024u;
    ++E;
  }
  if (E > 15) return 0x7C00;
  return (uint16_t)(((uint32_t)(E + 15) << 10) | (q - 1024u));
}

// Sum of one int64 per thread over the workgroup (result on thread 0).
__device__ __forceinline__ int64_t block_sum64(int64_t v, int64_t* part) {
  const int t = threadIdx.x;
  part[t] = v;
  __syncthreads();
  for (int w = kSign2Threads / 2; w > 0; w >>= 1) {
    if (t < w) part[t] += part[t + w];
    __syncthreads();
  }
  const int64_t r = part[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kSign2Threads) void pack_sign2_kernel(
    const uint16_t* __restrict__ w, int rows, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales) {
  __shared__ int64_t part[kSign2Threads];
  const int t = threadIdx.x;
  const int64_t col = blockIdx.x;
  const uint16_t* src = w + col * rows;
  // s0: mean magnitude
  int64_t acc = 0;
  for (int i = t; i < rows; i += kSign2Threads) {
    const int64_t v = h_units(src[i]);
    acc += v < 0 ? -v : v;
  }
  const int64_t S0 = block_sum64(acc, part);
  const uint16_t s0h = f64_to_h_rne(ldexp((double)S0 / (double)rows, -24));
  const int64_t s0 = h_units(s0h);
  // s1: mean magnitude of the residual of the first sign code
  acc = 0;
  for (int i = t; i < rows; i += kSign2Threads) {
    const int64_t v = h_units(src[i]);
    const int64_t r = v - (v >= 0 ? s0 : -s0);
    acc += r < 0 ? -r : r;
  }
  const int64_t S1 = block_sum64(acc, part);
  const uint16_t s1h = f64_to_h_rne(ldexp((double)S1 / (double)rows, -24));
  const int64_t s1 = h_units(s1h);
  if (t == 0) {
    scales[2 * col] = s0h;
    scales[2 * col + 1] = s1h;
  }
  // codes: levels in code order u = 0..3 are (+,+), (+,-), (-,+), (-,-);
  // the first minimum (smallest u) wins
  const int64_t L[4] = {s0 + s1, s0 - s1, -s0 + s1, -s0 - s1};
  for (int b = t; b < rows / 4; b += kSign2Threads) {
    uint32_t byte = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t v = h_units(src[4 * b + r]);
      uint32_t best = 0;
      int64_t bd = v - L[0] < 0 ? L[0] - v : v - L[0];
#pragma unroll
      for (uint32_t k = 1; k < 4; ++k) {
        const int64_t d = v - L[k] < 0 ? L[k] - v : v - L[k];
        if (d < bd) {
          bd = d;
          best = k;
        }
      }
      byte |= best << (2 * r);
    }
    codes[col * (rows / 4) + b] = (uint8_t)byte;
  }
}

// ---------------------------------------------------------------------------
// Trellis encoder on the GPU (offline). SpAx page section 5.1: per column a
// sequence of 2-bit codes minimising the squared error between the weights
// divided by their root-mean-square and codebook[window], chosen jointly by
// the Viterbi algorithm. The arithmetic is the host encoder's, operation by
// operation (so both give the same codes): the exact sum of squares in
// 128-bit integers, one rounding each for S -> fp64, / rows, sqrt, -> fp16;
// fp32 errors without contraction; the smallest dropped code and then the
// smallest final state win ties.
// One 1024-thread workgroup per column; thread T owns the 16 trellis states
// 16T .. 16T+15, whose predecessors are the 64 consecutive states
// 64 (T mod 256) .. +63 and whose windows are codebook[64T .. 64T+63] (kept in
// registers). Each row: read the 64 predecessor costs, barrier, write the 16
// new costs and one 32-bit word of backpointers (2 bits per state) to the
// workspace, barrier. Thread 0 then traces the best path back.
// ---------------------------------------------------------------------------
constexpr int kTrelThreads = 1024;
constexpr int kTrelStates = 1 << 14;
constexpr int kTrelVChunk = 1024;

struct U128 {
  uint64_t hi, lo;
};
__device__ __forceinline__ U128 add128(U128 a, U128 b) {
  const uint64_t lo = a.lo + b.lo;
  return U128{a.hi + b.hi + (lo < a.lo ? 1u : 0u), lo};
}
// u * u for u < 2^40
__device__ __forceinline__ U128 square40(uint64_t u) {
  const uint64_t uh = u >> 32, ul = u & 0xFFFFFFFFu;
  const uint64_t ll = ul * ul;        // < 2^64
  const uint64_t hl = 2u * uh * ul;   // < 2^41
  const uint64_t hh = uh * uh;        // < 2^16
  U128 r{hh, ll};
  return add128(r, U128{hl >> 32, hl << 32});
}
// round a 128-bit unsigned integer to fp64, ties to even
__device__ __forceinline__ double u128_to_f64(U128 v) {
  if (v.hi == 0) return (double)v.lo;  // u64 -> f64, one rounding
  const int n = 128 - __builtin_clzll(v.hi);  // significant bits, > 64
  const int sh = n - 53;                      // 12 .. 75
  uint64_t mant, rem_hi, rem_lo, half_hi, half_lo;
  if (sh < 64) {
    mant = (v.hi << (64 - sh)) | (v.lo >> sh);
    rem_hi = 0;
    rem_lo = v.lo & ((uint64_t(1) << sh) - 1);
    half_hi = 0;
    half_lo = uint64_t(1) << (sh - 1);
  } else {
    mant = v.hi >> (sh - 64);
    rem_hi = sh == 64 ? 0 : v.hi & ((uint64_t(1) << (sh - 64)) - 1);
    rem_lo = v.lo;
    half_hi = sh == 64 ? 0 : uint64_t(1) << (sh - 65);
    half_lo = sh == 64 ? uint64_t(1) << 63 : 0;
  }
  const bool above = rem_hi > half_hi || (rem_hi == half_hi && rem_lo > half_lo);
  const bool tie = rem_hi == half_hi && rem_lo == half_lo;
  if (above || (tie && (mant & 1u))) ++mant;  // 2^53 stays exact in fp64
  return ldexp((double)mant, sh);
}

__global__ __launch_bounds__(kTrelThreads) void trellis_encode_kernel(
    const uint16_t* __restrict__ w, int rows, int col0, const uint16_t* __restrict__ cb,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, uint32_t* __restrict__ bp) {
#pragma clang fp contract(off)
  // two cost buffers (row i reads one, writes the other); the reductions
  // before and after the trellis borrow them
  __shared__ __attribute__((aligned(16))) float cost[2][kTrelStates];
  __shared__ float vbuf[kTrelVChunk];
  const int t = threadIdx.x;
  const int64_t col = col0 + (int64_t)blockIdx.x;
  const uint16_t* src = w + col * rows;
  uint32_t* bpc = bp + (int64_t)blockIdx.x * rows * kTrelThreads;
  uint64_t* rhi = reinterpret_cast<uint64_t*>(&cost[0][0]);
  uint64_t* rlo = rhi + kTrelThreads;

  // scale: exact sum of squares, then one rounding per step
  U128 acc{0, 0};
  for (int i = t; i < rows; i += kTrelThreads) {
    const int64_t u = h_units(src[i]);
    acc = add128(acc, square40((uint64_t)(u < 0 ? -u : u)));
  }
  rhi[t] = acc.hi;
  rlo[t] = acc.lo;
  __syncthreads();
  for (int k = kTrelThreads / 2; k > 0; k >>= 1) {
    if (t < k) {
      const U128 r = add128(U128{rhi[t], rlo[t]}, U128{rhi[t + k], rlo[t + k]});
      rhi[t] = r.hi;
      rlo[t] = r.lo;
    }
    __syncthreads();
  }
  const double q = u128_to_f64(U128{rhi[0], rlo[0]}) / (double)rows;
  const uint16_t sh = f64_to_h_rne(ldexp(sqrt(q), -24));
  __syncthreads();  // the reduction's words are read; cost[0] is free again
  if (t == 0) scales[col] = sh;
  uint8_t* cc = codes + col * (rows / 4);
  if (sh == 0) {
    for (int b = t; b < rows / 4; b += kTrelThreads) cc[b] = 0;
    return;
  }
  const double s = ldexp((double)h_units(sh), -24);

  // this thread's 64 windows as fp16 pairs; d = v - cb is taken as the
  // fused fp16 x fp32 + fp32 operation fma(cb, -1, v): one rounding of the
  // exact difference, as an fp32 subtraction
  uint32_t cbp[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    cbp[k] = (uint32_t)cb[64 * t + 2 * k] | ((uint32_t)cb[64 * t + 2 * k + 1] << 16);
  const float inf = __builtin_inff();
#pragma unroll
  for (int k = 0; k < 16; ++k) cost[0][16 * t + k] = (t == 0 && k == 0) ? 0.0f : inf;
  const int pbase = 64 * (t & 0xFF);
  int cur = 0;

  for (int c0 = 0; c0 < rows; c0 += kTrelVChunk) {
    const int cn = min(kTrelVChunk, rows - c0);
    __syncthreads();
    for (int i = t; i < cn; i += kTrelThreads)
      vbuf[i] = (float)(ldexp((double)h_units(src[c0 + i]), -24) / s);
    __syncthreads();
    for (int i = 0; i < cn; ++i) {
      const float v = vbuf[i];
      const float* pc = cost[cur];
      float* nx = cost[cur ^ 1];
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 q4 = *reinterpret_cast<const float4*>(&pc[pbase + 4 * k]);
        const float pk[4] = {q4.x, q4.y, q4.z, q4.w};
        float best = 0.0f;
        uint32_t bo = 0;
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          const uint32_t pair = cbp[2 * k + (o >> 1)];
          const float cbo = h2f((uint16_t)((o & 1) ? pair >> 16 : pair & 0xFFFFu));
          const float d = fmaf(cbo, -1.0f, v);
          const float e = d * d;
          const float c = pk[o] + e;
          if (o == 0 || c < best) {
            best = c;
            bo = (uint32_t)o;
          }
        }
        nx[16 * t + k] = best;
        bits |= bo << (2 * k);
      }
      bpc[(int64_t)(c0 + i) * kTrelThreads + t] = bits;
      cur ^= 1;
      __syncthreads();
    }
  }

  // the best final state (smallest cost, then smallest state)
  float bv = cost[cur][16 * t];
  int bi = 16 * t;
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    const float c = cost[cur][16 * t + k];
    if (c < bv) {
      bv = c;
      bi = 16 * t + k;
    }
  }
  float* rv = cost[cur ^ 1];
  int32_t* ri = reinterpret_cast<int32_t*>(rv + kTrelThreads);
  rv[t] = bv;
  ri[t] = bi;
  __syncthreads();
  for (int k = kTrelThreads / 2; k > 0; k >>= 1) {
    if (t < k) {
      const float o = rv[t + k];
      const int oi = ri[t + k];
      if (o < rv[t] || (o == rv[t] && oi < ri[t])) {
        rv[t] = o;
        ri[t] = oi;
      }
    }
    __syncthreads();
  }
  // trace back (thread 0): the code of row i is the state's top two bits
  if (t == 0) {
    int state = ri[0];
    uint32_t byte = 0;
    for (int i = rows - 1; i >= 0; --i) {
      byte |= ((uint32_t)state >> 12) << (2 * (i & 3));
      if ((i & 3) == 0) {
        cc[i >> 2] = (uint8_t)byte;
        byte = 0;
      }
      const uint32_t word = bpc[(int64_t)i * kTrelThreads + (state >> 4)];
      state = ((state & 0xFFF) << 2) | (int)((word >> (2 * (state & 15))) & 3u);
    }
  }
}

// Squared l2 distance of two fp16 vectors, added to (or stored in) one fp64
// value: one workgroup; thread t sums the terms t, t + 1024, ... in order,
// then a fixed tree over the threads (the same bits on every call).
constexpr int kSqThreads = 1024;
__global__ __launch_bounds__(kSqThreads) void sq_error_kernel(const uint16_t* __restrict__ y,
                                                              const uint16_t* __restrict__ r,
                                                              int64_t n, double* acc,
                                                              int accumulate) {
  __shared__ double part[kSqThreads];
  const int t = (int)threadIdx.x;
  double s = 0.0;
  for (int64_t i = t; i < n; i += kSqThreads) {
    const double d = (double)h2f(y[i]) - (double)h2f(r[i]);  // exact in fp64
    s = fma(d, d, s);
  }
  part[t] = s;
  __syncthreads();
  for (int h = kSqThreads / 2; h > 0; h >>= 1) {
    if (t < h) part[t] += part[t + h];
    __syncthreads();
  }
  if (t == 0) *acc = accumulate ? *acc + part[0] : part[0];
}

__global__ void clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  const int64_t cols = (int64_t)(a.f_hi - a.f_lo) + (a.a_hi - a.a_lo);
  if (cols <= 0) return hipSuccess;
  const int64_t waves = (kCopyThreads / 64);
  int64_t blocks = (cols + waves - 1) / waves;
  if (blocks > 512) blocks = 512;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, int32_t rows, int32_t cols, int32_t fmt,
                       uint8_t* codes, uint16_t* scales, hipStream_t s) {
  const int64_t items = (int64_t)cols * (rows / kGroup);
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 3) / 4;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, rows, cols, fmt,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_sign2(const uint16_t* w, int32_t rows, int32_t cols, uint8_t* codes,
                             uint16_t* scales, hipStream_t s) {
  if (cols == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_sign2_kernel, dim3((unsigned)cols), dim3(kSign2Threads), 0, s, w,
                     rows, codes, scales);
  return hipGetLastError();
}

size_t trellis_ws_per_column(int32_t rows) { return (size_t)rows * kTrelThreads * 4; }

hipError_t launch_pack_trellis(const uint16_t* w, int32_t rows, int32_t cols,
                               const uint16_t* codebook, uint8_t* codes, uint16_t* scales,
                               void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t batch = std::min<int64_t>(cols, (int64_t)(ws_bytes / trellis_ws_per_column(rows)));
  for (int64_t c0 = 0; c0 < cols; c0 += batch) {
    const int64_t nb = std::min<int64_t>(batch, cols - c0);
    hipLaunchKernelGGL(trellis_encode_kernel, dim3((unsigned)nb), dim3(kTrelThreads), 0, s, w,
                       rows, (int)c0, codebook, codes, scales, static_cast<uint32_t*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sq_error(const uint16_t* y, const uint16_t* r, int64_t n, double* acc,
                           int32_t accumulate, hipStream_t s) {
  hipLaunchKernelGGL(sq_error_kernel, dim3(1), dim3(kSqThreads), 0, s, y, r, n, acc,
                     (int)accumulate);
  return hipGetLastError();
}

hipError_t launch_clear(void* ws, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(ws), n);
  return hipGetLastError();
}

}  // namespace spax
