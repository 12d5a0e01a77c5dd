// Device helpers shared by the tiered-product kernels: fp16 bit helpers,
// buffer resources, and the in-workgroup tier selection (SpAx page, section
// 5, Figure 2 step 3: rank x by |x_j|, the largest k_full go to the full
// tier, the next k_approx to the approx tier).
#pragma once

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

// Per-format load and multiply-add of one lane's 8 consecutive rows of one
// column: fp16 values (16 bytes), int4 codes (4 bytes) or int2 codes
// (2 bytes). offset(row0, lane) is the byte offset, within a column, of
// row row0 + 8 * lane.
template <int FMT>
struct Tier;

template <>
struct Tier<kFp16> {
  using V = uint4;
  // columns per round (a round's loads stay in registers, double-buffered)
  static constexpr int U = kWaves > 8 ? 4 : 8;
  // byte offset of lane l's 8 rows in a column
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return 2u * (uint32_t)(row0 + 8 * lane);
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t, off, col, 0));
  }
  static constexpr float kScale = 1.0f;
  static constexpr uint32_t kMask = 0u;
  // f = x_j
  static __device__ __forceinline__ void fma(float (&acc)[8], float&, V v, float f, uint32_t) {
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

// Code tiers: each code u is turned into the fp16 value 1 + u / 2^b (b the
// code width; the code fills the top mantissa bits under the exponent of
// 1.0), two rows per 32-bit word, and multiplied in by fp16 x fp32 FMAs
// (v_fma_mix_f32) -- no int-to-float conversions. The factor f passed in is
// 2^b x_j s_{j,g} (kScale; exact), so each FMA adds x_j s (2^b + u); the
// running sum corr takes back x_j s (2^b + the code offset) per column.
template <>
struct Tier<kInt4> {
  using V = uint32_t;
  static constexpr int U = 8;
  static constexpr float kScale = 16.0f;  // 2^4
  static constexpr uint32_t kMask = 0x03C003C0u;  // bits 6..9 of both halves
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 2u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_amdgcn_raw_buffer_load_b32(t, off, col, 0);
  }
  // Row k sits in nibble k (bits 4k..4k+3) as two's-complement q; flipping
  // each nibble's sign bit gives u = q + 8. Rows k and k+4 land in bits
  // 6..9 of the two halves with one shift: fp16 1 + u/16.
  // Adds x s (16 + u); corr takes back x s (16 + 8) = 1.5 f. kM is kMask
  // held in a VGPR, so each pair is one shift and one v_and_or_b32.
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float f,
                                             uint32_t kM) {
    corr = fmaf(1.5f, f, corr);
    v ^= 0x88888888u;
    constexpr uint32_t kOne = 0x3C003C00u;
    const uint32_t p0 = ((v << 6) & kM) | kOne;  // rows 0, 4
    const uint32_t p1 = ((v << 2) & kM) | kOne;  // rows 1, 5
    const uint32_t p2 = ((v >> 2) & kM) | kOne;  // rows 2, 6
    const uint32_t p3 = ((v >> 6) & kM) | kOne;  // rows 3, 7
    acc[0] = fmaf(h2f(p0 & 0xFFFFu), f, acc[0]);
    acc[4] = fmaf(h2f(p0 >> 16), f, acc[4]);
    acc[1] = fmaf(h2f(p1 & 0xFFFFu), f, acc[1]);
    acc[5] = fmaf(h2f(p1 >> 16), f, acc[5]);
    acc[2] = fmaf(h2f(p2 & 0xFFFFu), f, acc[2]);
    acc[6] = fmaf(h2f(p2 >> 16), f, acc[6]);
    acc[3] = fmaf(h2f(p3 & 0xFFFFu), f, acc[3]);
    acc[7] = fmaf(h2f(p3 >> 16), f, acc[7]);
  }
};

template <>
struct Tier<kInt2> {
  using V = uint32_t;
  static constexpr int U = 8;
  static constexpr float kScale = 4.0f;  // 2^2
  static constexpr uint32_t kMask = 0x03000300u;  // bits 8..9 of both halves
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 4u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_amdgcn_raw_buffer_load_b16(t, off, col, 0);
  }
  // Row 4b + r sits in bits 2r..2r+1 of byte b (two bytes per lane). The
  // second byte moves to bits 16..23; then rows r and 4 + r land in bits
  // 8..9 of the two halves with one shift: fp16 1 + u/4.
  // Adds x s (4 + u); corr takes back x s (4 + 1.5) = 1.375 f. kM is kMask
  // held in a VGPR, so each pair is one shift and one v_and_or_b32.
  static __device__ __forceinline__ void fma(float (&acc)[8], float& corr, V v, float f,
                                             uint32_t kM) {
    corr = fmaf(1.375f, f, corr);
    const uint32_t w = (v & 0xFFu) | ((v & 0xFF00u) << 8);
    constexpr uint32_t kOne = 0x3C003C00u;
    const uint32_t p0 = ((w << 8) & kM) | kOne;  // rows 0, 4
    const uint32_t p1 = ((w << 6) & kM) | kOne;  // rows 1, 5
    const uint32_t p2 = ((w << 4) & kM) | kOne;  // rows 2, 6
    const uint32_t p3 = ((w << 2) & kM) | kOne;  // rows 3, 7
    acc[0] = fmaf(h2f(p0 & 0xFFFFu), f, acc[0]);
    acc[4] = fmaf(h2f(p0 >> 16), f, acc[4]);
    acc[1] = fmaf(h2f(p1 & 0xFFFFu), f, acc[1]);
    acc[5] = fmaf(h2f(p1 >> 16), f, acc[5]);
    acc[2] = fmaf(h2f(p2 & 0xFFFFu), f, acc[2]);
    acc[6] = fmaf(h2f(p2 >> 16), f, acc[6]);
    acc[3] = fmaf(h2f(p3 & 0xFFFFu), f, acc[3]);
    acc[7] = fmaf(h2f(p3 >> 16), f, acc[7]);
  }
};

// The SpAx page's two-scale sign code (section 5.1, Eq. 4): weight i of
// column j is e1 s_{j,0} + e2 s_{j,1}. Row 4b + r holds [e2 = -1] in bit 2r
// and [e1 = -1] in bit 2r + 1 of byte b (two bytes per lane). The second
// byte moves to bits 16..23; each sign bit of rows r and r + 4 is then
// shifted into the sign bits (15 and 31) of a pair of fp16 1.0s, and the
// resulting +-1 are multiplied in by fp16 x fp32 FMAs with the column's
// factors fa = x_j s_{j,0} and fb = x_j s_{j,1}. Every added term is exactly
// +-x_j s, with no offset to take back. kM is kMask held in a VGPR.
template <>
struct Tier<kSign2> {
  using V = uint32_t;
  static constexpr int U = 8;
  static constexpr uint32_t kMask = 0x80008000u;  // sign bits of both halves
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 4u;
  }
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t t, uint32_t off, uint32_t col) {
    return __builtin_amdgcn_raw_buffer_load_b16(t, off, col, 0);
  }
  static __device__ __forceinline__ void fma2(float (&acc)[8], V v, float fa, float fb,
                                              uint32_t kM) {
    const uint32_t w = (v & 0xFFu) | ((v & 0xFF00u) << 8);
    constexpr uint32_t kOne = 0x3C003C00u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t pa = ((w << (14 - 2 * r)) & kM) | kOne;  // e1 of rows r, r + 4
      const uint32_t pb = ((w << (15 - 2 * r)) & kM) | kOne;  // e2 of rows r, r + 4
      acc[r] = fmaf(h2f(pa & 0xFFFFu), fa, acc[r]);
      acc[r] = fmaf(h2f(pb & 0xFFFFu), fb, acc[r]);
      acc[r + 4] = fmaf(h2f(pa >> 16), fa, acc[r + 4]);
      acc[r + 4] = fmaf(h2f(pb >> 16), fb, acc[r + 4]);
    }
  }
};

// The SpAx page's trellis-coded middle tier (section 5.1, trellis coding):
// weight i of column j is cb[index_i] s_j with index_i the window of the
// 2-bit codes of rows i-7..i of the same matrix column (oldest code in the
// low bits; codes before the column start are zero). Lane l holds the codes
// of its rows 8l..8l+7 in the high half of V and those of the 8 rows before
// them in the low half (the streaming code loads both; in a stored column
// that holds several matrices the rows before come from the same matrix),
// so row 8l + r reads its window with one bit-field extract, then one LDS
// lookup into the codebook and one fp16 x fp32 FMA with the column's factor
// x_j s_j.
template <>
struct Tier<kTrellis> {
  using V = uint32_t;  // codes of rows 8l-8 .. 8l+7, two bits each
  // 4 columns per round: each column takes two loads (the lane's rows and
  // the 8 rows before them in the same matrix), and 8 columns per round
  // spilled registers (7B attention: 16.5 against 17.8 us per launch)
  static constexpr int U = 4;
  static constexpr uint32_t kMask = 0u;
  static __device__ __forceinline__ uint32_t offset(int row0, int lane) {
    return (uint32_t)(row0 + 8 * lane) / 4u;
  }
  static __device__ __forceinline__ void fma_cb(float (&acc)[8], V v, float f,
                                                const uint16_t* cb) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t index = (v >> (2 * r + 2)) & 0xFFFFu;
      acc[r] = fmaf(h2f(cb[index]), f, acc[r]);
    }
  }
};

// ---------------------------------------------------------------------------
// In-workgroup tier selection (kListRank). Same definition as the stand-alone
// plan kernel: order key = fp16 magnitude bits, larger first, lower index
// first among equal keys; the k_full first are F, the next k_approx are A.
// The histogram steps run on the first kRankWaves waves only (the other
// waves meet the barriers): they are issue-bound, a few instructions per
// entry plus a fixed cost per wave and step, so fewer waves over more
// entries each take less time per SIMD. The counting and placement steps
// run on every wave over its own short chunk, since only the threads whose
// positions meet the piece place entries, and a long per-thread loop there
// would leave one wave with all the work. Entries past n read as key 0 and
// are taken out of the counts of key 0 where the boundaries are found;
// they are never placed.
//   1. 256-bin histogram of key bits 14..7;
//   2. suffix counts give the bins holding rank k_full and k_full + k_approx;
//   3. 128-bin histograms inside those two bins (one pass) give the boundary
//      keys t1, t2 and the number of entries equal to each that are kept
//      (q1, q2);
//   4. one scan of (#key > t1, #key == t1, #key > t2, #key == t2) over the
//      workgroup, packed two counts per register, gives every entry its
//      position: #F before entry i is gt1(i) + min(eq1(i), q1), #(F or A)
//      before it gt2(i) + min(eq2(i), q2).
// Histograms keep kHistCopies interleaved copies of each bin (lane l adds
// to copy l mod kHistCopies), so skewed inputs (many equal magnitudes, e.g.
// exact zeros) put at most 64 / kHistCopies adds of one instruction on one
// LDS address.
// ---------------------------------------------------------------------------
constexpr uint32_t kAboveAll = 0x8000u;  // boundary key when a tier is empty
// Measured on the 7B attention launches: 8 ranking waves (two per SIMD)
// beat 4 by 0.2-0.3 us per launch; the ranking waves then overlap each
// other's LDS and barrier waits.
constexpr int kRankWaves = 8;
constexpr int kRankThreads = kRankWaves * 64;
constexpr int kHistCopies = 4;
static_assert(kRankWaves <= kWaves && kRankMaxN % (kRankThreads * 32) == 0,
              "fused ranking entries per thread are multiples of 8");

struct RankShared {
  // bin b, copy c at word kHistCopies * b + c
  uint32_t hist[256 * kHistCopies];
  // sub-bins in the bin of rank k_full at [0, 128), in the bin of rank
  // k_full + k_approx at [128, 256) (both at [0, 128) when the bins coincide)
  uint32_t sub[256 * kHistCopies];
  uint32_t spare[64];  // per-lane targets of the adds that count nothing
  uint32_t scan[2][kWaves];  // packed count pairs, per wave
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

// Inclusive prefix sum within each 16-lane row (row shifts only).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
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

// Adds E per-entry bins (-1: not counted) to an LDS histogram, one entry
// per thread at a time. When the whole wave holds the same bin, one lane
// adds 64 at once: skewed inputs (many equal magnitudes, e.g. exact zeros)
// then do not serialise 64 atomics on one LDS address.
template <int E, class BinOf>
__device__ __forceinline__ void hist_add(uint32_t* hist, BinOf bin_of) {
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int b = bin_of(i);
    const int b0 = __builtin_amdgcn_readfirstlane(b);
    if (__ballot(b == b0) == ~0ull) {  // wave-uniform
      if (b0 >= 0 && (threadIdx.x & 63) == 0) atomicAdd(&hist[b0], 64u);
    } else if (b >= 0) {
      atomicAdd(&hist[b], 1u);
    }
  }
}

__device__ __forceinline__ uint32_t rawbits(const uint32_t* xr, int i) {
  return (xr[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

// Loads entries [base, base + C) of x as raw fp16 bits, two per register,
// 0 past n: 16-byte loads, or 8-byte ones where C is not a multiple of 8
// (x is 16-byte aligned and base a multiple of C).
template <int C>
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ x, int n, int base,
                                           uint32_t* r) {
  static_assert(C % 4 == 0, "chunk of whole 8-byte words");
  constexpr int L = C % 8 == 0 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < C; i += L) {
    if (base + i + L - 1 < n) {
      if constexpr (L == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + base + i);
        r[i / 2 + 0] = v.x;
        r[i / 2 + 1] = v.y;
        r[i / 2 + 2] = v.z;
        r[i / 2 + 3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(x + base + i);
        r[i / 2 + 0] = v.x;
        r[i / 2 + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < L; j += 2) {
        const uint32_t lo = base + i + j < n ? x[base + i + j] : 0u;
        const uint32_t hi = base + i + j + 1 < n ? x[base + i + j + 1] : 0u;
        r[(i + j) / 2] = lo | (hi << 16);
      }
    }
  }
}

// 15-bit key (fp16 magnitude pattern) of entry i of a packed chunk
__device__ __forceinline__ uint32_t chunk_key(const uint32_t* r, int i) {
  return (i & 1) ? (r[i >> 1] >> 16) & 0x7FFFu : r[i >> 1] & 0x7FFFu;
}

// Ranks x and places this workgroup's list positions in LDS: full-tier
// positions [f0, f1) at slots [0, f1 - f0), approx-tier positions [a0, a1)
// after them. Every thread owns the chunk [t*C, t*C + C) of x, C = E *
// kRankThreads / kGemvThreads, for the counting and placement steps;
// ranking thread t builds the histograms from the chunks of threads t,
// t + kRankThreads, ... (E entries).
template <int E>
__device__ __forceinline__ void rank_piece(const GemvArgs& a, RankShared& rs, int32_t* lidx,
                                           float* lx, int f0, int f1, int a0, int a1,
                                           bool write_lists) {
  constexpr int kChunks = kGemvThreads / kRankThreads;
  constexpr int C = E / kChunks;
  static_assert(E % kChunks == 0 && C % 4 == 0, "whole 8-byte words per chunk");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const bool ranker = t < kRankThreads;  // wave-uniform
  const int n = a.n;
  const int base = t * C;
  const uint32_t K1 = (uint32_t)a.k_full;
  const uint32_t K2 = (uint32_t)(a.k_full + a.k_approx);
  const uint32_t pad = (uint32_t)(kGemvThreads * C - n);  // entries past n
  const uint32_t copy = (uint32_t)(lane & (kHistCopies - 1));

  uint32_t xp[C / 2];                   // this thread's chunk
  uint32_t xq[(kChunks - 1) * C / 2];   // a ranking thread's other chunks
  load_chunk<C>(a.x, n, base, xp);
  if (ranker) {
#pragma unroll
    for (int c = 1; c < kChunks; ++c)
      load_chunk<C>(a.x, n, (t + c * kRankThreads) * C, xq + (c - 1) * (C / 2));
  }
  // key of a ranking thread's entry i of E
  auto rkey = [&](int i) -> uint32_t { return i < C ? chunk_key(xp, i) : chunk_key(xq, i - C); };

  // both histograms cleared at once (2 words per thread)
  static_assert(2 * 256 * kHistCopies == 2 * kGemvThreads, "one 8-byte clear per thread");
  reinterpret_cast<uint2*>(rs.hist)[t] = make_uint2(0u, 0u);
  __syncthreads();

  // 1. top-level histogram
  if (ranker) {
#pragma unroll
    for (int i = 0; i < E; ++i) atomicAdd(&rs.hist[((rkey(i) >> 7) << 2) | copy], 1u);
  }
  __syncthreads();

  // 2. bins holding rank K1 and rank K2 (1-based, from the largest key),
  // found by wave 0; the padding is taken out of bin 0
  if (wave == 0) {
    uint32_t c[4];
    const uint4* hp = reinterpret_cast<const uint4*>(rs.hist) + 4 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = hp[j];
      c[j] = v.x + v.y + v.z + v.w;
    }
    if (lane == 0) c[0] -= pad;
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

  // 3. low-level histograms inside the two boundary bins, in one pass;
  // other entries add to the lane's spare word
  const int b1 = rs.sel[0];
  const int b2 = rs.sel[2];
  const int b2x = b2 == b1 ? -1 : b2;  // a shared bin is counted once
  if (ranker) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t k = rkey(i);
      const int hb = (int)(k >> 7);
      const uint32_t w = ((k & 127u) << 2) | copy;
      uint32_t* p = hb == b1 ? &rs.sub[w]
                             : (hb == b2x ? &rs.sub[128 * kHistCopies + w] : &rs.spare[lane]);
      atomicAdd(p, 1u);
    }
  }
  __syncthreads();
  // boundary keys t (kAboveAll when the tier is empty) and quotas q: the
  // number of entries equal to t that are kept; found by wave 0
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = r == 0 ? b1 : b2;
      const uint32_t K = r == 0 ? K1 : K2;
      int key_t = (int)kAboveAll;
      uint32_t quota = 0u;
      if (b >= 0) {  // wave-uniform
        const uint4* sp = reinterpret_cast<const uint4*>(
                              rs.sub + (r == 1 && b2x >= 0 ? 128 * kHistCopies : 0)) +
                          2 * lane;
        const uint4 v0 = sp[0], v1 = sp[1];
        uint32_t c0 = v0.x + v0.y + v0.z + v0.w, c1 = v1.x + v1.y + v1.z + v1.w;
        if (b == 0 && lane == 0) c0 -= pad;  // the padding has key 0
        uint32_t above = (uint32_t)rs.sel[1 + 2 * r] + wave_excl_suffix(c0 + c1);
        int sk = -1;
        uint32_t sq = 0u;
        if (above < K && K <= above + c1) { sk = (b << 7) | (2 * lane + 1); sq = K - above; }
        above += c1;
        if (above < K && K <= above + c0) { sk = (b << 7) | (2 * lane); sq = K - above; }
        wave_pick(sk, sq, key_t, quota);
      }
      if (lane == 0) {
        rs.sel[4 + 2 * r] = key_t;
        rs.sel[5 + 2 * r] = (int32_t)quota;
      }
    }
  }
  __syncthreads();
  const uint32_t t1 = (uint32_t)rs.sel[4], q1 = (uint32_t)rs.sel[5];
  const uint32_t t2 = (uint32_t)rs.sel[6], q2 = (uint32_t)rs.sel[7];

  // 4. positions, every thread over its chunk. The padding (key 0, after
  // every real entry) may be counted as equal to a boundary key 0, but the
  // quota of such a key is used up by the real zeros before it, so it is
  // never placed.
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const uint32_t k = chunk_key(xp, i);
    c[0] += k > t1;
    c[1] += k == t1;
    c[2] += k > t2;
    c[3] += k == t2;
  }
  // Scans run on the counts packed two per register: every partial sum
  // below is under 2^16 (at most kRankMaxN), and the packed sums subtract
  // exactly.
  static_assert(kWaves <= 16, "wave totals fit one 16-lane row");
  const uint32_t p01 = c[0] | (c[1] << 16), p23 = c[2] | (c[3] << 16);
  const uint32_t i01 = wave_incl_scan(p01), i23 = wave_incl_scan(p23);
  if (lane == 63) {
    rs.scan[0][wave] = i01;
    rs.scan[1][wave] = i23;
  }
  __syncthreads();
  // totals of the waves before this one: lane 16 h + w holds wave w's total
  // of pair h; a scan within each 16-lane row gives the prefixes
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t wt = (lane >> 4) < 2 && (lane & 15) < kWaves ? rs.scan[lane >> 4][lane & 15] : 0u;
  const uint32_t wex = row16_incl_scan(wt) - wt;
  const uint32_t ex01 = (uint32_t)__builtin_amdgcn_readlane((int)wex, wv) + i01 - p01;
  const uint32_t ex23 = (uint32_t)__builtin_amdgcn_readlane((int)wex, 16 + wv) + i23 - p23;
  uint32_t g1 = ex01 & 0xFFFFu, e1r = ex01 >> 16;
  uint32_t g2 = ex23 & 0xFFFFu, e2r = ex23 >> 16;
  // This thread's F positions [fs, fe) and A positions [as, ae); only
  // threads whose positions meet the piece place entries.
  const int fs = (int)(g1 + min(e1r, q1));
  const int fe = (int)(g1 + c[0] + min(e1r + c[1], q1));
  const int as = (int)(g2 + min(e2r, q2)) - fs;
  const int ae = (int)(g2 + c[2] + min(e2r + c[3], q2)) - fe;
  if ((fs < f1 && fe > f0) || (as < a1 && ae > a0)) {
    const int nf = f1 - f0;
    // fresh copies of the boundary keys: the comparisons below are not
    // shared with the counting above (sharing them kept 4C compare masks
    // alive across the barrier)
    uint32_t t1c = t1, t2c = t2;
    asm volatile("" : "+v"(t1c), "+v"(t2c));
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const uint32_t k = chunk_key(xp, i);
      const bool gt1 = k > t1c, eq1 = k == t1c, gt2 = k > t2c, eq2 = k == t2c;
      const bool in_f = gt1 || (eq1 && e1r < q1);
      const bool in_fa = gt2 || (eq2 && e2r < q2);
      const int fpos = (int)(g1 + min(e1r, q1));          // F entries before this one
      const int apos = (int)(g2 + min(e2r, q2)) - fpos;   // A entries before this one
      const bool put_f = in_f && fpos >= f0 && fpos < f1;
      const bool put_a = in_fa && !in_f && apos >= a0 && apos < a1;
      const int slot = put_f ? fpos - f0 : nf + (apos - a0);
      if (put_f || put_a) {
        lidx[slot] = base + i;
        lx[slot] = h2f((i & 1) ? xp[i >> 1] >> 16 : xp[i >> 1] & 0xFFFFu);
      }
      g1 += gt1;
      e1r += eq1;
      g2 += gt2;
      e2r += eq2;
    }
  }
  __syncthreads();
  // the caller's lists: this piece, copied out of LDS
  if (write_lists) {
    const int nf = f1 - f0;
    for (int q = t; q < nf; q += kGemvThreads) a.out_full_idx[f0 + q] = lidx[q];
    for (int q = t; q < a1 - a0; q += kGemvThreads) a.out_approx_idx[a0 + q] = lidx[nf + q];
  }
}

// Places this workgroup's piece (full-tier positions [f0, f1) at LDS slots
// [0, f1 - f0), approx-tier positions [a0, a1) after them) from the sliced
// selection's thresholds and per-slice counts: only the slices whose
// positions meet the piece are scanned, 4 entries per thread. The same
// position rule as rank_piece.
__device__ __forceinline__ void place_sliced(const GemvArgs& a, uint32_t (&scan_sm)[2][kWaves],
                                             int32_t* lidx, float* lx, int f0, int f1, int a0,
                                             int a1, bool write_lists) {
  const SelectScratch* ws = a.sel;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int n = a.n;
  const uint32_t t1 = (uint32_t)ws->sel[4], q1 = (uint32_t)ws->sel[5];
  const uint32_t t2 = (uint32_t)ws->sel[6], q2 = (uint32_t)ws->sel[7];
  const int nf = f1 - f0;
  // counts of the slices before the current one
  uint32_t G1 = 0u, E1 = 0u, G2 = 0u, E2 = 0u;
  for (int s = 0; s < a.slices; ++s) {
    const uint32_t c0 = ws->cnt[s][0], c1 = ws->cnt[s][1];
    const uint32_t c2 = ws->cnt[s][2], c3 = ws->cnt[s][3];
    const int fs = (int)(G1 + min(E1, q1)), fe = (int)(G1 + c0 + min(E1 + c1, q1));
    const int as = (int)(G2 + min(E2, q2)) - fs, ae = (int)(G2 + c2 + min(E2 + c3, q2)) - fe;
    if ((fs < f1 && fe > f0) || (as < a1 && ae > a0)) {  // wave-uniform
      const int base = s * kSliceEntries + 4 * t;
      uint32_t xr[2];
      if (base + 3 < n) {
        const uint2 v = *reinterpret_cast<const uint2*>(a.x + base);
        xr[0] = v.x;
        xr[1] = v.y;
      } else {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const uint32_t lo = base + j < n ? a.x[base + j] : 0u;
          const uint32_t hi = base + j + 1 < n ? a.x[base + j + 1] : 0u;
          xr[j / 2] = lo | (hi << 16);
        }
      }
      const int nv = max(0, min(4, n - base));
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = rawbits(xr, i) & 0x7FFFu;
        const bool ok = i < nv;
        c[0] += ok && k > t1;
        c[1] += ok && k == t1;
        c[2] += ok && k > t2;
        c[3] += ok && k == t2;
      }
      // in-slice prefixes, packed two counts per register (under 2^16)
      const uint32_t p01 = c[0] | (c[1] << 16), p23 = c[2] | (c[3] << 16);
      const uint32_t i01 = wave_incl_scan(p01), i23 = wave_incl_scan(p23);
      if (lane == 63) {
        scan_sm[0][wave] = i01;
        scan_sm[1][wave] = i23;
      }
      __syncthreads();
      const uint32_t wt =
          (lane >> 4) < 2 && (lane & 15) < kWaves ? scan_sm[lane >> 4][lane & 15] : 0u;
      const uint32_t wex = row16_incl_scan(wt) - wt;
      const uint32_t ex01 = (uint32_t)__builtin_amdgcn_readlane((int)wex, wv) + i01 - p01;
      const uint32_t ex23 = (uint32_t)__builtin_amdgcn_readlane((int)wex, 16 + wv) + i23 - p23;
      uint32_t g1 = G1 + (ex01 & 0xFFFFu), e1r = E1 + (ex01 >> 16);
      uint32_t g2 = G2 + (ex23 & 0xFFFFu), e2r = E2 + (ex23 >> 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = rawbits(xr, i) & 0x7FFFu;
        const bool ok = i < nv;
        const bool gt1 = ok && k > t1, eq1 = ok && k == t1;
        const bool gt2 = ok && k > t2, eq2 = ok && k == t2;
        const bool in_f = gt1 || (eq1 && e1r < q1);
        const bool in_fa = gt2 || (eq2 && e2r < q2);
        const int fpos = (int)(g1 + min(e1r, q1));
        const int apos = (int)(g2 + min(e2r, q2)) - fpos;
        const bool put_f = in_f && fpos >= f0 && fpos < f1;
        const bool put_a = in_fa && !in_f && apos >= a0 && apos < a1;
        const int slot = put_f ? fpos - f0 : nf + (apos - a0);
        if (put_f || put_a) {
          lidx[slot] = base + i;
          lx[slot] = h2f(rawbits(xr, i));
        }
        g1 += gt1;
        e1r += eq1;
        g2 += gt2;
        e2r += eq2;
      }
      __syncthreads();  // scan_sm is reused by the next slice
    }
    G1 += c0;
    E1 += c1;
    G2 += c2;
    E2 += c3;
  }
  __syncthreads();
  if (write_lists) {
    for (int q = t; q < nf; q += kGemvThreads) a.out_full_idx[f0 + q] = lidx[q];
    for (int q = t; q < a1 - a0; q += kGemvThreads) a.out_approx_idx[a0 + q] = lidx[nf + q];
  }
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

}  // namespace
}  // namespace spax
