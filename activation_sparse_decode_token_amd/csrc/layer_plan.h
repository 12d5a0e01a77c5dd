// Work schedule of the layer kernel: one launch runs every group of a
// decoder layer (SpAx page, section 5.2: q/k/v share the ranking of their
// input, o has its own, gate/up share one, down ranks a = silu(g) * u).
// Shared by the host (planning, the schedule export) and the kernel.
//
// Phases. The gate/up group comes first (down needs all of its output), then
// q/k/v and o, then down. A group runs on a contiguous range of workgroups:
// gate/up and down on all of them; q/k/v and o split the workgroups in
// proportion to their bytes (each of the two on all of them when the other
// is absent).
//
// Units. Group g with T row tiles and K = k_full + k_approx selected columns
// has U = T K units, unit u being list position u mod K of tile u / K. Its
// workgroups take equal runs of units: workgroup i of the group's n_wg takes
// [U i / n_wg, U (i + 1) / n_wg). A run's part of tile t is a position range
// [q0, q1); it takes the full-tier list positions [q0 k_full / K,
// q1 k_full / K) and the approx-tier positions [q0 k_approx / K,
// q1 k_approx / K) of that tile, so consecutive runs partition each tier's
// list exactly and every run holds both tiers in the same proportion (the
// same mix of bytes and dequantisation work). K is at most 32768, so every
// product here fits 32 bits.
//
// Partial sums. Workgroup i's sum for tile t goes to slot t + i of the
// group's partials: along the unit line (t, i) pairs are ordered, so t + i is
// strictly increasing and below T + n_wg. The workgroups that meet tile t are
// those whose runs hold units t K and (t + 1) K - 1 and every one between.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "spax.h"
#include "spax_internal.h"

namespace spax {

// Waves of one layer-kernel workgroup: streaming waves, one reduction wave,
// then the ranking waves.
constexpr int kLayerStreamWaves = 11;
constexpr int kLayerReduceWave = kLayerStreamWaves;
constexpr int kLayerRankWaves = 4;
constexpr int kLayerRankThreads = kLayerRankWaves * 64;
static_assert(kLayerStreamWaves + 1 + kLayerRankWaves == kWaves, "16 waves");
// List entries (16-bit column indices) of every present group, kept in LDS
// for the whole launch.
constexpr int kLayerListCap = 20480;
// Longest input the ranking waves rank: its keys sit in LDS during a
// ranking (32768 fp16 keys, 64 KB).
constexpr int kLayerMaxN = 32768;
// Entries of one ranking round (one wave: 64 lanes x 8 keys).
constexpr int kRankRound = 512;
constexpr int kRankMaxRounds = kLayerMaxN / kRankRound;
// Most workgroups of one launch (the partial-sum region is sized for it).
constexpr int kLayerMaxWgs = 512;
// Most segments one workgroup meets in one phase (its LDS segment table);
// the host runs the layer kernel only when every workgroup stays within it.
constexpr int kLayerSegTab = 160;

// One group of the layer (indexed by the public group id).
struct LayerGroupArgs {
  int32_t present;          // the group runs in this launch
  int32_t rows;             // stored rows R
  int32_t n;                // input length
  int32_t k_full, k_approx;
  int32_t tiles;            // ceil(R / 512)
  int32_t list_off;         // LDS entry offset of the group's lists (F then A)
  int32_t wg_lo, n_wg;      // the group's workgroups [wg_lo, wg_lo + n_wg)
  uint32_t units;           // tiles * (k_full + k_approx) (0: no columns)
  uint32_t unit_q, unit_r;  // units = unit_q * n_wg + unit_r
  uint32_t k_magic;         // div_magic(k_full + k_approx)
  uint32_t nwg_magic;       // div_magic(n_wg)
  const uint8_t* full_base;
  int64_t full_stride;
  uint32_t full_bytes;
  uint32_t approx_bytes;
  const uint16_t* full_scales;
  int64_t full_sstride;
  const uint8_t* approx_base;
  int64_t approx_stride;
  const uint16_t* approx_scales;
  int64_t approx_sstride;
  int32_t approx_seg, approx_nseg;  // matrices per stored column (as GemvArgs)
  const uint16_t* x;        // the group's input (down: the a gate/up writes)
  uint16_t* y;              // plain output (null for gate/up)
  int32_t* out_full;        // the caller's tier lists
  int32_t* out_approx;
  float* partials;          // [tiles + n_wg][512] fp32
  uint32_t* counters;       // tile t at counters[t * kCountersPerTile]
};

struct LayerArgs {
  LayerGroupArgs g[4];
  int32_t order[4];         // present groups in processing order
  int32_t n_order;
  int32_t G;                // workgroups
  int32_t down_waits;       // down's input is written by this launch's gate/up
  uint16_t* glu_a;
  uint16_t* glu_g;          // optional
  uint16_t* glu_u;          // optional
  // [0] gate/up tiles complete, [1] workgroups finished, [2] status bits
  uint32_t* sync;
};

// One workgroup's work on one row tile of one group.
struct LayerSeg {
  int32_t g;                // public group id
  int32_t t;                // row tile
  int32_t f0, f1;           // full-tier list positions
  int32_t a0, a1;           // approx-tier list positions
  int32_t w_lo, w_hi;       // the workgroups that meet this tile
};

// Processing order of the groups (absent ones are skipped): gate/up first,
// down last.
__host__ __device__ constexpr int layer_order(int oi) {
  return oi == 0 ? SPAX_GROUP_GATE_UP : oi == 1 ? SPAX_GROUP_QKV : oi == 2 ? SPAX_GROUP_O
                                                                          : SPAX_GROUP_DOWN;
}

// Division by a divisor fixed for the launch: m = div_magic(d) =
// floor(2^32 / d) (2^32 - 1 for d = 1) makes floor(a m / 2^32) equal
// floor(a / d) or one less (a m / 2^32 lies in (a / d - 1, a / d]), which
// one comparison corrects. The kernel's schedule arithmetic then costs a
// multiply instead of a full 32-bit division.
inline uint32_t div_magic(uint32_t d) {
  return d <= 1u ? 0xFFFFFFFFu : (uint32_t)((uint64_t(1) << 32) / d);
}
__host__ __device__ inline uint32_t div_by(uint32_t a, uint32_t d, uint32_t m) {
  uint32_t q = (uint32_t)(((uint64_t)a * m) >> 32);
  if ((uint64_t)(q + 1u) * d <= a) ++q;
  return q;
}

// First unit of run i of a group: floor(U i / n) with U = q n + r, as
// q i + floor(r i / n) (r i below 2^18).
__host__ __device__ inline uint32_t layer_run_start(const LayerGroupArgs& gr, uint32_t i) {
  return gr.unit_q * i + div_by(gr.unit_r * i, (uint32_t)gr.n_wg, gr.nwg_magic);
}

// The workgroup (index within the group) whose run holds unit u:
// floor(((u + 1) n - 1) / U), by a double-precision estimate and one exact
// correction (the numerator is below 2^41, the quotient below 2^9).
__host__ __device__ inline uint32_t layer_run_of(const LayerGroupArgs& gr, uint32_t u) {
  const uint64_t a = (uint64_t)(u + 1u) * (uint32_t)gr.n_wg - 1u, b = gr.units;
  uint64_t q = (uint64_t)((double)a / (double)b);
  if (q * b > a)
    --q;
  else if ((q + 1) * b <= a)
    ++q;
  return (uint32_t)q;
}

// Whether workgroup w works on group g.
__host__ __device__ inline bool layer_meets(const LayerArgs& A, int g, uint32_t w) {
  const LayerGroupArgs& gr = A.g[g];
  if (!gr.present) return false;
  if (gr.units == 0) return w < (uint32_t)gr.tiles;
  return w >= (uint32_t)gr.wg_lo && w < (uint32_t)(gr.wg_lo + gr.n_wg);
}

// The tiles of group g that workgroup w meets: t_first, t_first + step, ...
// below t_end, and w's run [u0, u1) of the group's units. False when w does
// not work on g.
__host__ __device__ inline bool layer_group_range(const LayerArgs& A, int g, uint32_t w,
                                                  uint32_t& t_first, uint32_t& step,
                                                  uint32_t& t_end, uint32_t& u0, uint32_t& u1) {
  const LayerGroupArgs& gr = A.g[g];
  if (!gr.present) return false;
  u0 = u1 = 0u;
  if (gr.units == 0) {
    t_first = w;
    step = (uint32_t)A.G;
    t_end = (uint32_t)gr.tiles;
    return t_first < t_end;
  }
  if (w < (uint32_t)gr.wg_lo || w >= (uint32_t)(gr.wg_lo + gr.n_wg)) return false;
  const uint32_t i = w - (uint32_t)gr.wg_lo;
  const uint32_t K = (uint32_t)(gr.k_full + gr.k_approx);
  u0 = layer_run_start(gr, i);
  u1 = layer_run_start(gr, i + 1);
  t_first = div_by(u0, K, gr.k_magic);
  step = 1u;
  t_end = div_by(u1 + K - 1u, K, gr.k_magic);
  return t_first < t_end;
}

// Workgroup w's segment of tile t of group g (its run [u0, u1)), with
// w_lo = w_hi = -1 unless the group has no selected columns (the contributors
// are found by layer_contributors).
__host__ __device__ inline LayerSeg layer_make_seg(const LayerArgs& A, int g, uint32_t w,
                                                   uint32_t t, uint32_t u0, uint32_t u1) {
  const LayerGroupArgs& gr = A.g[g];
  LayerSeg s;
  s.g = g;
  s.t = (int32_t)t;
  if (gr.units == 0) {
    s.f0 = s.f1 = s.a0 = s.a1 = 0;
    s.w_lo = s.w_hi = (int32_t)w;
  } else {
    const uint32_t K = (uint32_t)(gr.k_full + gr.k_approx);
    const uint32_t q0 = (u0 > t * K ? u0 - t * K : 0u);
    const uint32_t q1 = (u1 < (t + 1) * K ? u1 - t * K : K);
    s.f0 = (int32_t)div_by(q0 * (uint32_t)gr.k_full, K, gr.k_magic);
    s.f1 = (int32_t)div_by(q1 * (uint32_t)gr.k_full, K, gr.k_magic);
    s.a0 = (int32_t)div_by(q0 * (uint32_t)gr.k_approx, K, gr.k_magic);
    s.a1 = (int32_t)div_by(q1 * (uint32_t)gr.k_approx, K, gr.k_magic);
    s.w_lo = s.w_hi = -1;
  }
  return s;
}

// Calls f(seg) for each segment of workgroup w in group g, in tile order.
// A group with no selected columns (units 0) still writes its output: its
// tiles are dealt to the workgroups round-robin as empty one-contributor
// segments.
template <class F>
__host__ __device__ inline void layer_group_segs(const LayerArgs& A, int g, uint32_t w, F f) {
  uint32_t t, step, t_end, u0, u1;
  if (!layer_group_range(A, g, w, t, step, t_end, u0, u1)) return;
  // one call site of f (its body is large in the kernel)
  for (; t < t_end; t += step) f(layer_make_seg(A, g, w, t, u0, u1));
}

// Resumable walk over workgroup w's segments of the groups selected by a
// predicate, in processing order.
struct LayerCursor {
  int32_t oi;
  uint32_t t, step, t_end, u0, u1;
};

__host__ __device__ inline void layer_cursor_init(LayerCursor& c) {
  c.oi = -1;
  c.t = c.t_end = 0u;
  c.step = 1u;
  c.u0 = c.u1 = 0u;
}

template <class Pred>
__host__ __device__ inline bool layer_cursor_next(const LayerArgs& A, uint32_t w, Pred take,
                                                  LayerCursor& c, LayerSeg& s) {
  while (c.t >= c.t_end) {
    if (++c.oi >= A.n_order) return false;
    const int g = A.order[c.oi];
    c.t = c.t_end = 0u;
    if (!take(g)) continue;
    if (!layer_group_range(A, g, w, c.t, c.step, c.t_end, c.u0, c.u1)) c.t = c.t_end = 0u;
  }
  s = layer_make_seg(A, A.order[c.oi], w, c.t, c.u0, c.u1);
  c.t += c.step;
  return true;
}

// The first and last workgroup that meet tile s.t of group s.g.
__host__ __device__ inline void layer_contributors(const LayerArgs& A, LayerSeg& s) {
  const LayerGroupArgs& gr = A.g[s.g];
  if (gr.units == 0) return;  // one contributor, set by layer_group_segs
  const uint32_t K = (uint32_t)(gr.k_full + gr.k_approx);
  s.w_lo = gr.wg_lo + (int32_t)layer_run_of(gr, (uint32_t)s.t * K);
  s.w_hi = gr.wg_lo + (int32_t)layer_run_of(gr, ((uint32_t)s.t + 1u) * K - 1u);
}

// An upper bound on the segments any workgroup meets in the phase of the
// groups selected by take: per group, the tiles a run of ceil(U / n_wg)
// units can touch (or, with no selected columns, the tiles dealt
// round-robin).
template <class Pred>
inline uint32_t layer_phase_segs_bound(const LayerArgs& A, Pred take) {
  uint32_t b = 0;
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    const LayerGroupArgs& gr = A.g[g];
    if (!take(g)) continue;
    if (gr.units == 0) {
      b += ((uint32_t)gr.tiles + (uint32_t)A.G - 1u) / (uint32_t)A.G;
    } else {
      const uint32_t K = (uint32_t)(gr.k_full + gr.k_approx);
      const uint32_t run = (gr.units + (uint32_t)gr.n_wg - 1u) / (uint32_t)gr.n_wg;
      const uint32_t t = (run + K - 2u) / K + 1u;
      b += t < (uint32_t)gr.tiles ? t : (uint32_t)gr.tiles;
    }
  }
  return b;
}

hipError_t launch_layer(const LayerArgs& a, int32_t full_fmt, int32_t approx_fmt,
                        hipStream_t s);

}  // namespace spax
