// Per-wave streaming of one tier's selected columns (gfx950), shared by the
// per-projection product (gemv.hip) and the layer kernel (layer.hip).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "block_common.h"
#include "spax_internal.h"

namespace spax {
namespace {

// Factors of one wave's current 64-column batch of a code tier, in LDS:
// x_j * s_{j,g} for each 128-row group g of the tile (0 past the batch).
struct WaveMeta {
  float fac[64][4];
};

// Makes this wave's LDS writes visible to all its lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// One wave's stream over list positions [p_lo, p_hi) of one tier, for its
// rows of the tile. Batches of 64 columns: lane l fetches position p + l
// (kListGlobal: index list and activations in device memory; kListStaged:
// staging position, activation via the index list; kListRank: the
// workgroup's piece in LDS) and keeps the column and activation in
// registers; each column's index (and an fp16 column's activation) reaches
// the wave with readlane. Code tiers form x_j * s_{j,g} per lane and group
// in LDS, since each lane needs the factor of its own 128-row group.
// Rounds of U columns are double-buffered: the loads of round r + 1 are
// issued before round r is consumed, so a wave always has a round in
// flight. Slots past the batch reload its last column and are not added,
// which keeps every load unconditional.
// begin() issues the first round early -- before the other tier is
// streamed -- so the two tiers' first loads share one memory latency. The
// code loads of a batch are issued before its scales have arrived; the
// factors are formed just before the batch is consumed.
template <int FMT, int MODE>
struct TierStream {
  using T = Tier<FMT>;
  using V = typename T::V;
  static constexpr int U = T::U;
  // group-scaled integer codes: a factor per 128-row group, through LDS
  static constexpr bool kCode = FMT == kInt4 || FMT == kInt2;
  // two-scale sign code: two factors per column, lane-uniform (readlane)
  static constexpr bool kTwo = FMT == kSign2;
  // trellis code: one factor per column (readlane), codebook in LDS
  static constexpr bool kTrel = FMT == kTrellis;

  WaveMeta& wm;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off, cstride;
  int gsel, ngrp, row0, lane;
  const uint16_t* __restrict__ scales;
  int64_t sstride;
  const int32_t* __restrict__ idx;
  const uint16_t* __restrict__ x;
  const int32_t* lidx;
  const float* lx;
  int p_lo, p_hi;
  V v0[U];
  uint32_t vmask;  // the tier's code mask, kept in a VGPR
  int mycol;       // this lane's column of the pending batch
  float xv;        // this lane's activation of the pending batch (0 past it)
  float xb;        // sign code: x_j s_{j,1} (xv then holds x_j s_{j,0})
  const uint16_t* cbk = nullptr;  // trellis code: the codebook in LDS
  // Sign / trellis codes of stored columns that hold several matrices (each
  // coded as its own column): the tile holds rows of at most two of them,
  // seg_a and seg_b (GLU gate and up; one stacked matrix when equal); the
  // lane's rows belong to seg_b when seg_sel is set. xv1 / xb1 are the
  // factors of seg_b.
  int seg_a = 0, seg_b = 0;
  bool seg_sel = false, two_segs = false;
  float xv1 = 0.0f, xb1 = 0.0f;
  // Trellis code: byte offset of the lane's 8 rows before (in the same
  // matrix) and whether there are any (none at a matrix's first row).
  uint32_t boff = 0u;
  bool has_before = false;
  uint32_t sc[4];  // this lane's raw fp16 scales of the pending batch (codes)

  __device__ __forceinline__ TierStream(WaveMeta& wm_, const uint8_t* base, int64_t stride,
                                        uint32_t bytes, const uint16_t* scales_, int64_t sstride_,
                                        const int32_t* idx_, const uint16_t* x_,
                                        const int32_t* lidx_, const float* lx_, int p_lo_,
                                        int p_hi_, int row0_, int rows, int lane_, int ld_lane,
                                        int seg_mode = 0)
      : wm(wm_), rs(tier_rsrc(base, bytes)), off(T::offset(row0_, ld_lane)),
        cstride((uint32_t)stride), gsel(kCode ? (ld_lane >> 4) : 0),
        ngrp(min(4, (rows - row0_ + kGroup - 1) / kGroup)), row0(row0_), lane(lane_),
        scales(scales_), sstride(sstride_), idx(idx_), x(x_), lidx(lidx_), lx(lx_),
        p_lo(p_lo_), p_hi(p_hi_) {
    // opaque to the optimiser: the mask stays in a VGPR instead of becoming
    // a literal (gfx9 VOP3 instructions take no literals)
    vmask = T::kMask;
    asm volatile("" : "+v"(vmask));
    if constexpr (kTwo || kTrel) {
      const int r = row0_ + 8 * ld_lane;  // the lane's first row
      if (seg_mode < 0) {                 // GLU: gate blocks even, up blocks odd
        seg_a = 0;
        seg_b = 1;
        two_segs = true;
        seg_sel = ((r >> 7) & 1) != 0;
      } else if (seg_mode > 0) {          // stacked: the tile lies in one matrix
        seg_a = seg_b = row0_ / seg_mode;
      }
      if constexpr (kTrel) {
        // the 8 rows before the lane's rows, in the same matrix: the previous
        // 8 stored rows, or in the GLU layout at a 128-row block start the
        // last 8 rows of the matrix's previous block (256 stored rows back);
        // none at the matrix's first row
        if (seg_mode < 0 && (r & 127) == 0) {
          has_before = r >= 256;
          boff = has_before ? (uint32_t)(r - 136) / 4u : 0u;
        } else {
          has_before = seg_mode > 0 ? (r % seg_mode) != 0 : r != 0;
          boff = has_before ? (uint32_t)(r - 8) / 4u : 0u;
        }
      }
    }
  }

  // This lane's column and activation of the batch at pb, and (codes) its
  // raw scales, without waiting for the scales.
  __device__ __forceinline__ void fill_cols(int pb, int cnt) {
    xv = 0.0f;
    xb = 0.0f;
    xv1 = 0.0f;
    xb1 = 0.0f;
    mycol = 0;
    if (lane < cnt) {
      const int q = pb + lane;
      int j;
      if constexpr (MODE == kListRank || MODE == kListSliced) {
        j = lidx[q];
        xv = lx[q];
      } else if constexpr (MODE == kListPacked) {
        // the layer kernel's lists: 16-bit column indices in LDS; x_j read
        // coherently (down's input is written by the same launch)
        j = (int)reinterpret_cast<const uint16_t*>(lidx)[q];
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(x), (short)0, 0x7FFFFFFF, 0x00020000);
        xv = h2f(__builtin_amdgcn_raw_buffer_load_b16(xr, 2u * (uint32_t)j, 0, 16));
      } else {
        j = idx[q];
        xv = h2f(x[j]);
      }
      mycol = MODE == kListStaged ? q : j;
      if constexpr (kTrel) {  // x_j s_j of the tile's two matrices
        const uint16_t* sp = scales + (int64_t)mycol * sstride;
        xv1 = xv * h2f(sp[seg_b]);
        xv = xv * h2f(sp[seg_a]);
      }
      if constexpr (kTwo) {
        // each matrix's (s0, s1) in one 4-byte load
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(scales + (int64_t)mycol * sstride);
        const uint32_t sv = sp[seg_a], sv1 = sp[seg_b];
        xb1 = xv * h2f(sv1 >> 16);
        xv1 = xv * h2f(sv1 & 0xFFFFu);
        xb = xv * h2f(sv >> 16);
        xv = xv * h2f(sv & 0xFFFFu);
      }
      if constexpr (kCode) {
        const uint16_t* sp = scales + (int64_t)mycol * sstride + (row0 >> 7);
        if (ngrp == 4 && (sstride & 3) == 0) {
          // the tile's 4 group scales in one 8-byte load (aligned: row0 is
          // a multiple of 512 and a column's scales start 8-byte aligned)
          const uint2 v = *reinterpret_cast<const uint2*>(sp);
          sc[0] = v.x & 0xFFFFu;
          sc[1] = v.x >> 16;
          sc[2] = v.y & 0xFFFFu;
          sc[3] = v.y >> 16;
        } else {
          // a ragged last tile has fewer groups; their slots are never read
          // (lanes past the last row take group 0's rows)
          const int gl = ngrp - 1;
#pragma unroll
          for (int g = 0; g < 4; ++g) sc[g] = sp[min(g, gl)];
        }
      }
    }
  }
  // Code factors 2^b x_j s_{j,g} of the pending batch (0 past the batch).
  __device__ __forceinline__ void fill_facs(int cnt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) wm.fac[lane][g] = lane < cnt ? xv * h2f(sc[g]) * T::kScale : 0.0f;
    wave_sync();
  }
  __device__ __forceinline__ void issue(int r, int cnt, V (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(r * U + u, cnt - 1);
      const uint32_t col = (uint32_t)__builtin_amdgcn_readlane(mycol, c);
      if constexpr (kTrel) {
        // the lane's 8 rows (high half) after the 8 rows before them
        const uint32_t cur = __builtin_amdgcn_raw_buffer_load_b16(rs, off, col * cstride, 0);
        const uint32_t before = __builtin_amdgcn_raw_buffer_load_b16(rs, boff, col * cstride, 0);
        v[u] = (has_before ? before : 0u) | (cur << 16);
      } else {
        v[u] = T::load(rs, off, col * cstride);
      }
    }
  }
  // Adds batch column c (loaded as v) to the accumulators.
  __device__ __forceinline__ void add(float (&acc)[8], float& corr, int c, const V& v) {
    if constexpr (kTwo) {
      float fa = readlane_f(xv, c), fb = readlane_f(xb, c);
      if (two_segs) {  // wave-uniform
        const float fa1 = readlane_f(xv1, c), fb1 = readlane_f(xb1, c);
        fa = seg_sel ? fa1 : fa;
        fb = seg_sel ? fb1 : fb;
      }
      T::fma2(acc, v, fa, fb, vmask);
    } else if constexpr (kTrel) {
      float f = readlane_f(xv, c);
      if (two_segs) f = seg_sel ? readlane_f(xv1, c) : f;
      T::fma_cb(acc, v, f, cbk);
    }
    else
      T::fma(acc, corr, v, kCode ? wm.fac[c][gsel] : readlane_f(xv, c), vmask);
  }
  __device__ __forceinline__ void use(float (&acc)[8], float& corr, int r, int cnt,
                                      const V (&v)[U]) {
    if ((r + 1) * U <= cnt) {  // a full round (wave-uniform)
#pragma unroll
      for (int u = 0; u < U; ++u) add(acc, corr, r * U + u, v[u]);
    } else {  // the batch's last, partial round: only its columns are added
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = r * U + u;
        if (c < cnt) add(acc, corr, c, v[u]);
      }
    }
  }

  __device__ __forceinline__ void begin() {
    if (p_lo < p_hi) {
      const int cnt = min(64, p_hi - p_lo);
      fill_cols(p_lo, cnt);
      issue(0, cnt, v0);
    }
  }

  __device__ __forceinline__ void run(float (&acc)[8], float& corr) {
    for (int pb = p_lo; pb < p_hi; pb += 64) {
      const int cnt = min(64, p_hi - pb);
      if (pb != p_lo) {
        fill_cols(pb, cnt);
        issue(0, cnt, v0);
      }
      if constexpr (kCode) fill_facs(cnt);
      const int rounds = (cnt + U - 1) / U;
      V v1[U];
      for (int r = 0;;) {
        if (r + 1 < rounds) {
          issue(r + 1, cnt, v1);
          use(acc, corr, r, cnt, v0);
        } else {
          use(acc, corr, r, cnt, v0);
          break;
        }
        ++r;
        if (r + 1 < rounds) {
          issue(r + 1, cnt, v0);
          use(acc, corr, r, cnt, v1);
        } else {
          use(acc, corr, r, cnt, v1);
          break;
        }
        ++r;
      }
    }
  }
};

}  // namespace
}  // namespace spax
