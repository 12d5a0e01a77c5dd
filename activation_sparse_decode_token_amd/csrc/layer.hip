// Layer kernel (gfx950): every group of one decoder layer in one launch.
//
// SpAx page, section 2 (the seven projections and a = silu(W_gate x) * W_up
// x), section 5 Figure 2 steps 3-5 (rank the input by |x_j|, read the top
// tier in full and the middle tier from its codes, skip the rest) and
// section 5.2 (the groups that share one ranking: q/k/v on h, o on z,
// gate/up on x, down on a).
//
// One persistent workgroup per compute unit. Its 16 waves have three roles:
//   * waves 0..10 stream: for each segment of the schedule (layer_plan.h)
//     they read their share of the segment's selected columns (the same
//     per-format streaming as the per-projection product) and hand an fp32
//     partial of the tile's 512 rows to LDS;
//   * wave 11 reduces: it adds the 11 wave partials of each segment in a
//     fixed order, stores the workgroup's partial, counts the workgroup in
//     on the tile's arrival counter and, as the tile's last contributor,
//     adds the contributors' partials in workgroup order and writes the
//     output (with the SwiGLU epilogue for gate/up). The streaming waves
//     never wait on global memory round trips of the reduction;
//   * waves 12..15 rank: for each further group the workgroup meets they
//     rank the group's input (two-level radix select on the fp16 magnitude
//     key, lower index first among equal keys) and place the list positions
//     the workgroup reads into LDS, as 16-bit column indices. The lists of
//     the next group are ready before the streaming waves reach it.
// The first group a workgroup meets is ranked by all 16 waves before the
// roles begin. Down's input a is complete only when every gate/up tile is,
// so down runs in a second phase: once the workgroup's other groups are
// done, one wave waits for the count of finished gate/up tiles (a bounded
// wait), all 16 waves rank a, and the streaming and reduction waves run
// down's segments.
//
// Every wait is bounded. A wait that runs out sets a status bit in the
// workspace and goes on, so the launch always ends. Partial sums are added
// in an order fixed by the schedule, so results are bitwise reproducible.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "block_common.h"
#include "layer_plan.h"
#include "spax.h"
#include "spax_internal.h"
#include "stream_common.h"

namespace spax {
namespace {

constexpr int kNS = kLayerStreamWaves;
// Bounded waits: LDS flags (s_sleep 1 between polls) and the global count of
// finished gate/up tiles (one load round trip per poll).
constexpr uint32_t kSpinLds = 1u << 24;
constexpr uint32_t kSpinGlobal = 1u << 19;
constexpr uint32_t kStatusLdsWait = 1u;
constexpr uint32_t kStatusGlobalWait = 2u;
// Cache policy of coherent loads and stores (sc1): they reach the level
// shared by every XCD, like agent-scope atomics.
constexpr int kCoherent = 16;
// Contributors that share the final sum of a tile with many (second-phase
// down), and the rows each adds (one per lane).
constexpr uint32_t kFinalParts = 8;
constexpr int kPartRows = kTileRows / (int)kFinalParts;
static_assert(kPartRows == 64, "one row per lane");
static_assert(kCountersPerTile >= 8, "a free counter word per group");

struct LayerShared {
  uint16_t lists[kLayerListCap];             // every group's F then A lists
  uint16_t keys[kLayerMaxN];                 // ranking: the input's fp16 bits (the
                                             // four ranking waves), or the 32768-bin
                                             // key histogram (the whole workgroup)
  float slot[2][kNS][kTileRows];             // streaming waves' partials
  uint32_t hist[256 * kHistCopies];          // ranking: top-level histogram
  uint32_t sub[256 * kHistCopies];           // ranking: the two sub-histograms
  uint32_t rtot[kRankMaxRounds][4];          // ranking: per-round counts
  uint32_t wtot[kWaves];                     // ranking: per-wave histogram totals
  uint32_t rsel[4];                          // ranking: t1, q1, t2, q2
  uint32_t rsum[4];                          // ranking: the four counts over all rounds
  uint16_t spare[64];                        // ranking: per-lane target of unplaced entries
  uint32_t need[8];                          // ranking: positions to place
  uint32_t own[4];                           // ranking: positions to store out
  uint64_t rank_out[2];                      // ranking: the caller's lists
  uint4 segtab[kLayerSegTab];                // the phase's segments: g | t << 8,
                                             // f0 | f1 << 16, a0 | a1 << 16
  uint32_t nseg;                             // entries of segtab
  uint32_t ready[4];                         // a group's lists are in LDS
  uint32_t rbar;                             // ranking waves' barrier count
  uint32_t seg_arrive[2];                    // streaming-wave arrivals per slot set
  uint32_t seg_free;                         // segments whose slots were read
};
static_assert(sizeof(LayerShared) <= 160 * 1024, "LDS of one workgroup");

// The workgroup's LDS (one instance per launch of any layer kernel).
static __shared__ LayerShared g_sm;

// The LDS flags order LDS accesses only: their fences are restricted to
// LDS, so a wave's global loads in flight are not waited for (a full
// workgroup fence would wait for all of them).
__device__ __forceinline__ uint32_t lds_relaxed(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}
__device__ __forceinline__ void lds_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Adds v to the LDS counter p, after this wave's earlier LDS writes.
__device__ __forceinline__ void lds_signal_add(uint32_t* p, uint32_t v) {
  lds_release();
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Stores v to the LDS flag p, after this wave's earlier LDS accesses.
__device__ __forceinline__ void lds_signal_store(uint32_t* p, uint32_t v) {
  lds_release();
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// A barrier of the whole workgroup that orders its LDS accesses only: a
// full barrier would also wait for every global store the wave still has in
// flight (the ranking's tier lists to the caller, read by no one here).
__device__ __forceinline__ void lds_barrier() {
  lds_release();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bit) {
  __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the LDS word p reaches v (bounded).
__device__ __forceinline__ void wait_lds_ge(uint32_t* p, uint32_t v, uint32_t* status) {
  for (uint32_t it = 0; lds_relaxed(p) < v; ++it) {
    if (it >= kSpinLds) {
      if ((threadIdx.x & 63) == 0) set_status(status, kStatusLdsWait);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  lds_acquire();
}

// A pointer that is the same in every lane, moved to scalar registers (each
// 32-bit half through readfirstlane, widened without sign extension).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(lo | (hi << 32));
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Barrier of the ranking waves: the hardware barrier when every wave of the
// workgroup ranks, else an LDS count (bounded).
template <int RW>
__device__ __forceinline__ void rank_sync(uint32_t& epoch, uint32_t* status) {
  if constexpr (RW == kWaves) {
    __syncthreads();
  } else {
    epoch += RW;
    if ((threadIdx.x & 63) == 0) lds_signal_add(&g_sm.rbar, 1u);
    wait_lds_ge(&g_sm.rbar, epoch, status);
  }
}

// Histogram adds of the 8 keys in v (4 words, two fp16 patterns each).
__device__ __forceinline__ void hist8(const uint4& v, uint32_t copy) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t k = (w[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
    atomicAdd(&g_sm.hist[((k >> 7) << 2) | copy], 1u);
  }
}

// Counts over the 8 keys in v (fp16 magnitude bits): c1 = #(key > t1) |
// #(key == t1) << 16, c2 the same for t2.
__device__ __forceinline__ void lane_counts(const uint4& v, uint32_t t1, uint32_t t2,
                                            uint32_t& c1, uint32_t& c2) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  c1 = 0u;
  c2 = 0u;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t k = (w[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
    c1 += k > t1 ? 1u : (k == t1 ? 0x10000u : 0u);
    c2 += k > t2 ? 1u : (k == t2 ? 0x10000u : 0u);
  }
}


// What the placement of a ranking needs: the boundaries, the list positions
// the workgroup reads (two intervals per tier), the positions it stores to
// the caller's lists and their pointers (set_need).
struct Placement {
  uint32_t K1, t1, q1, t2, q2;
  uint32_t nf0, nf1, nf2, nf3, na0, na1, na2, na3;
  uint32_t of0, of1, oa0, oa1;
  int32_t* out_f;
  int32_t* out_a;
};

__device__ __forceinline__ Placement load_placement(uint32_t K1, uint32_t t1, uint32_t q1,
                                                    uint32_t t2, uint32_t q2) {
  const LayerShared& sm = g_sm;
  Placement P;
  P.K1 = K1; P.t1 = t1; P.q1 = q1; P.t2 = t2; P.q2 = q2;
  const uint4 nf = *reinterpret_cast<const uint4*>(&sm.need[0]);
  const uint4 na = *reinterpret_cast<const uint4*>(&sm.need[4]);
  P.nf0 = uniform(nf.x); P.nf1 = uniform(nf.y); P.nf2 = uniform(nf.z); P.nf3 = uniform(nf.w);
  P.na0 = uniform(na.x); P.na1 = uniform(na.y); P.na2 = uniform(na.z); P.na3 = uniform(na.w);
  const uint4 ow = *reinterpret_cast<const uint4*>(&sm.own[0]);
  P.of0 = uniform(ow.x); P.of1 = uniform(ow.y); P.oa0 = uniform(ow.z); P.oa1 = uniform(ow.w);
  P.out_f = uniform_ptr(reinterpret_cast<int32_t*>(sm.rank_out[0]));
  P.out_a = uniform_ptr(reinterpret_cast<int32_t*>(sm.rank_out[1]));
  return P;
}

// Whether a round whose counts before it are (G1, E1, G2, E2) and through it
// (G1e, E1e, G2e, E2e) holds a list position the workgroup needs.
__device__ __forceinline__ bool round_needed(const Placement& P, uint32_t G1, uint32_t E1,
                                             uint32_t G2, uint32_t E2, uint32_t G1e,
                                             uint32_t E1e, uint32_t G2e, uint32_t E2e) {
  // the round's full-tier and approx-tier position ranges
  const uint32_t fb = G1 + min(E1, P.q1), fe = G1e + min(E1e, P.q1);
  const uint32_t ab = G2 + min(E2, P.q2) - fb, ae = G2e + min(E2e, P.q2) - fe;
  return (fb < P.nf1 && fe > P.nf0) || (fb < P.nf3 && fe > P.nf2) ||
         (ab < P.na1 && ae > P.na0) || (ab < P.na3 && ae > P.na2);
}

// Places the lane's 8 entries e0 + h (keys v) of a round: x1, x2 are the
// lane's exclusive counts within the round (as lane_counts packs them),
// (G1, E1, G2, E2) the counts of the rounds before. Without branches: an
// entry of neither tier writes to its lane's spare slot, and a workgroup
// that stores positions to the caller's lists stores every entry through a
// buffer resource, at an offset past the list's end (a store the hardware
// drops) unless its position is one the workgroup owns.
__device__ __forceinline__ void place_round(const Placement& P, uint16_t* list, const uint4& v,
                                            uint32_t e0, uint32_t x1, uint32_t x2, uint32_t G1,
                                            uint32_t E1, uint32_t G2, uint32_t E2) {
  uint32_t g1 = G1 + (x1 & 0xFFFFu), e1 = E1 + (x1 >> 16);
  uint32_t g2 = G2 + (x2 & 0xFFFFu), e2 = E2 + (x2 >> 16);
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  const int lane = (int)threadIdx.x & 63;
  uint16_t* spare = &g_sm.spare[lane];
  const bool owner = P.of0 < P.of1 || P.oa0 < P.oa1;  // wave-uniform
  const __amdgpu_buffer_rsrc_t rf =
      tier_rsrc(reinterpret_cast<const uint8_t*>(P.out_f), 4u * P.of1);
  const __amdgpu_buffer_rsrc_t ra =
      tier_rsrc(reinterpret_cast<const uint8_t*>(P.out_a), 4u * P.oa1);
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t k = (w4[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
    const uint32_t fpos = g1 + min(e1, P.q1);
    const uint32_t apos = g2 + min(e2, P.q2) - fpos;
    // (an entry of F is also among the K2 largest: in_f implies in_fa)
    const bool in_f = k > P.t1 || (k == P.t1 && e1 < P.q1);
    const bool in_fa = k > P.t2 || (k == P.t2 && e2 < P.q2);
    const uint32_t e = e0 + (uint32_t)h;
    *(in_fa ? list + (in_f ? fpos : P.K1 + apos) : spare) = (uint16_t)e;
    if (owner) {
      const bool sf = in_f && fpos >= P.of0;
      const bool sa = !in_f && in_fa && apos >= P.oa0;
      __builtin_amdgcn_raw_buffer_store_b32(e, rf, sf ? 4u * fpos : 0xFFFFFFF0u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(e, ra, sa ? 4u * apos : 0xFFFFFFF0u, 0, 0);
    }
    g1 += k > P.t1 ? 1u : 0u;
    e1 += k == P.t1 ? 1u : 0u;
    g2 += k > P.t2 ? 1u : 0u;
    e2 += k == P.t2 ? 1u : 0u;
  }
}

// Ranks x[0, n) on RW waves (the last RW of the workgroup) and places the
// list positions this workgroup needs: the ascending F list (the K1 largest
// |x_j|) at list[0, K1) and the A list (the next K2 - K1) at list[K1, K2),
// one 16-bit column index per entry. The positions needed are g_sm.need:
// full-tier positions [need0, need1) and [need2, need3), approx-tier
// [need4, need5) and [need6, need7); placed entries at full-tier positions
// [own0, own1) and approx-tier [own2, own3) are also stored to the caller's
// lists (g_sm.rank_out). Keys go to LDS once, in rounds of 512 entries (round r on
// ranking wave r mod RW); entries past n are key 0 and are taken out of the
// counts of key 0 (they come after every real entry, so a boundary at key 0
// keeps real zeros first). Steps:
//   1. the keys into LDS and a 256-bin histogram of key bits 14..7 (4
//      interleaved copies per bin);
//   2. each ranking wave finds the bins b1, b2 holding ranks K1 and K2;
//   3. 128-bin histograms of key bits 6..0 inside b1 and b2;
//   4. each ranking wave finds the boundary keys t1, t2 and the numbers q1,
//      q2 of entries equal to them that are kept;
//   5. per round, the counts of key > t1, key == t1, key > t2, key == t2
//      (per-lane counts of its 8 entries, then a wave sum);
//   6. their exclusive scans over the rounds give each round's range of
//      list positions; in the rounds that meet a needed range, each lane
//      places its 8 entries (512 r + 8 l + h, h ascending) from its
//      exclusive counts within the round: #F before entry i is
//      gt1 + min(eq1, q1), #(F or A) before it gt2 + min(eq2, q2).
// The histograms are cleared again before the last barrier.
template <int RW>
__device__ __attribute__((noinline)) uint32_t rank_group(const uint16_t* __restrict__ x, int n,
                                                         uint32_t K1, uint32_t K2, int list_off,
                                                         uint32_t epoch, uint32_t* status) {
  // arguments of a call arrive in vector registers: make them scalar again
  x = uniform_ptr(x);
  n = (int)uniform((uint32_t)n);
  K1 = uniform(K1);
  K2 = uniform(K2);
  list_off = (int)uniform((uint32_t)list_off);
  epoch = uniform(epoch);
  LayerShared& sm = g_sm;
  uint16_t* list = sm.lists + list_off;
  const int rt = (int)threadIdx.x - (kWaves - RW) * 64;
  const int lane = rt & 63;
  const int rw = (int)uniform((uint32_t)(rt >> 6));
  const int R = (n + kRankRound - 1) / kRankRound;
  const uint32_t pad = (uint32_t)(R * kRankRound - n);  // key-0 entries past n
  const uint32_t copy = (uint32_t)(lane & (kHistCopies - 1));

  // 1. keys into LDS (plain loads: a launch's own down input is read only
  // after an agent-scope acquire), eight rounds of loads in flight per wave;
  // the round that holds the end of x is read entry by entry
  const __amdgpu_buffer_rsrc_t rs = tier_rsrc(reinterpret_cast<const uint8_t*>(x), 2u * n);
  const int Rfull = n / kRankRound;  // rounds entirely inside x
  for (int r0 = rw; r0 < Rfull; r0 += 8 * RW) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(r0 + u * RW, Rfull - 1);
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, 2u * (uint32_t)(r * kRankRound + 8 * lane), 0,
                                           0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * RW;
      if (r < Rfull) {
        *reinterpret_cast<uint4*>(&sm.keys[r * kRankRound + 8 * lane]) = v[u];
        hist8(v[u], copy);
      }
    }
  }
  if (Rfull < R && rw == Rfull % RW) {
    // the round that holds the end of x: loads past x's end (the buffer's
    // range) return 0, the padding's key, so no branch separates them
    const int e = Rfull * kRankRound + 8 * lane;
    uint32_t hw[8];
#pragma unroll
    for (int h = 0; h < 8; ++h)
      hw[h] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * (uint32_t)(e + h), 0, 0);
    const uint4 v = make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16),
                               hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16));
    *reinterpret_cast<uint4*>(&sm.keys[e]) = v;
    hist8(v, copy);
  }
  rank_sync<RW>(epoch, status);

  // 2. bins of rank K1 and rank K2 (1-based, from the largest key); the
  // padding is taken out of bin 0
  int b1, b2;
  uint32_t ab1, ab2;
  {
    uint32_t c4[4];
    const uint4* hp = reinterpret_cast<const uint4*>(sm.hist) + 4 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = hp[j];
      c4[j] = v.x + v.y + v.z + v.w;
    }
    if (lane == 0) c4[0] -= pad;
    uint32_t above = wave_excl_suffix(c4[0] + c4[1] + c4[2] + c4[3]);
    int s1 = -1, s2 = -1;
    uint32_t x1 = 0u, x2 = 0u;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (K1 > 0 && above < K1 && K1 <= above + c4[j]) { s1 = 4 * lane + j; x1 = above; }
      if (K2 > 0 && above < K2 && K2 <= above + c4[j]) { s2 = 4 * lane + j; x2 = above; }
      above += c4[j];
    }
    wave_pick(s1, x1, b1, ab1);
    wave_pick(s2, x2, b2, ab2);
  }

  // 3. sub-histograms inside the two boundary bins (a shared bin once)
  const int b2x = b2 == b1 ? -1 : b2;
  for (int r = rw; r < R; r += RW) {
    const uint4 v = *reinterpret_cast<const uint4*>(&sm.keys[r * kRankRound + 8 * lane]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t k = (w[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
      const int hb = (int)(k >> 7);
      const int off = hb == b1 ? 0 : (hb == b2x ? 128 * kHistCopies : -1);
      if (off >= 0) atomicAdd(&sm.sub[off + (int)(((k & 127u) << 2) | copy)], 1u);
    }
  }
  rank_sync<RW>(epoch, status);

  // 4. boundary keys (kAboveAll for an empty tier) and quotas; the padding
  // out of sub-bin 0
  uint32_t t1 = kAboveAll, q1 = 0u, t2 = kAboveAll, q2 = 0u;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int b = r == 0 ? b1 : b2;
    const uint32_t K = r == 0 ? K1 : K2;
    const uint32_t ab = r == 0 ? ab1 : ab2;
    if (b >= 0) {  // wave-uniform
      const uint4* sp =
          reinterpret_cast<const uint4*>(sm.sub + (r == 1 && b2x >= 0 ? 128 * kHistCopies : 0)) +
          2 * lane;
      const uint4 v0 = sp[0], v1 = sp[1];
      uint32_t c0 = v0.x + v0.y + v0.z + v0.w;
      const uint32_t c1 = v1.x + v1.y + v1.z + v1.w;
      if (b == 0 && lane == 0) c0 -= pad;
      uint32_t above = ab + wave_excl_suffix(c0 + c1);
      int sk = -1;
      uint32_t sq = 0u;
      if (above < K && K <= above + c1) { sk = (b << 7) | (2 * lane + 1); sq = K - above; }
      above += c1;
      if (above < K && K <= above + c0) { sk = (b << 7) | (2 * lane); sq = K - above; }
      int kt;
      uint32_t qt;
      wave_pick(sk, sq, kt, qt);
      if (r == 0) { t1 = (uint32_t)kt; q1 = qt; } else { t2 = (uint32_t)kt; q2 = qt; }
    }
  }
  t1 = uniform(t1); q1 = uniform(q1); t2 = uniform(t2); q2 = uniform(q2);

  // 5. per-round counts of key > t1, key == t1, key > t2, key == t2: each
  // lane counts its 8 entries (two counts per register), a wave sum gives
  // the round's
  for (int r = rw; r < R; r += RW) {
    const uint4 v = *reinterpret_cast<const uint4*>(&sm.keys[r * kRankRound + 8 * lane]);
    uint32_t c1, c2;
    lane_counts(v, t1, t2, c1, c2);
    c1 = wave_incl_scan(c1);
    c2 = wave_incl_scan(c2);
    if (lane == 63)
      *reinterpret_cast<uint4*>(&sm.rtot[r][0]) =
          make_uint4(c1 & 0xFFFFu, c1 >> 16, c2 & 0xFFFFu, c2 >> 16);
  }
  rank_sync<RW>(epoch, status);

  // 6. exclusive scans of the four counts over the rounds (lane l holds
  // round l), the needed rounds, then placement: lane l of round r places
  // its entries 512 r + 8 l + h in order, from the counts before it
  static_assert(kRankMaxRounds <= 64, "one round per lane");
  uint32_t ex[4], inc[4];
  {
    const uint4 u = lane < R ? *reinterpret_cast<const uint4*>(&sm.rtot[lane][0])
                             : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t own[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      inc[q] = wave_incl_scan(own[q]);
      ex[q] = inc[q] - own[q];
    }
  }
  const Placement P = load_placement(K1, t1, q1, t2, q2);
  for (int r = rw; r < R; r += RW) {
    const uint32_t G1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[0], r));
    const uint32_t E1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[1], r));
    const uint32_t G2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[2], r));
    const uint32_t E2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[3], r));
    const uint32_t G1e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[0], r));
    const uint32_t E1e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[1], r));
    const uint32_t G2e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[2], r));
    const uint32_t E2e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[3], r));
    if (!round_needed(P, G1, E1, G2, E2, G1e, E1e, G2e, E2e)) continue;  // wave-uniform
    const uint4 v = *reinterpret_cast<const uint4*>(&sm.keys[r * kRankRound + 8 * lane]);
    uint32_t c1, c2;
    lane_counts(v, t1, t2, c1, c2);
    place_round(P, list, v, (uint32_t)(r * kRankRound + 8 * lane), wave_incl_scan(c1) - c1,
                wave_incl_scan(c2) - c2, G1, E1, G2, E2);
  }
  static_assert(256 * kHistCopies == 4 * kLayerRankThreads, "one 16-byte clear per thread");
  if (rt < kLayerRankThreads) {
    reinterpret_cast<uint4*>(sm.hist)[rt] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(sm.sub)[rt] = make_uint4(0u, 0u, 0u, 0u);
  }
  rank_sync<RW>(epoch, status);
  return epoch;
}

// Ranks x[0, n) with the same result as rank_group (the same K1 largest
// |x_j| in F, the next K2 - K1 in A, lower index first among equal keys) and
// places the list positions this workgroup needs, on RW waves: the whole
// workgroup (RW = 16, nothing streams beside it) or the four ranking waves
// beside the streaming waves (RW = 4, inputs up to 4 rounds per wave). A
// wave gets one instruction per four cycles, and the ranking waves' issue
// cycles slow the streaming waves that share their SIMDs, so this variant
// spends as few instructions as it can: each wave's keys stay in registers
// (at most 4 rounds of 512 entries per wave) and an exact histogram of all
// 32768 keys sits in the keys' LDS area, which removes rank_group's second
// histogram pass and both bin searches. Steps:
//   1. the keys into registers (rounds rw, rw + RW, ...), the histogram
//      cleared meanwhile, then one LDS add per real entry (two 16-bit bins
//      per word: no bin exceeds n <= 32768, nor does any sum of bins below);
//   2. ranking thread i holds bins [B i, B i + B) (B = 32768 / (64 RW)): its
//      total, a suffix sum over the threads (a wave scan, then the waves'
//      totals) gives the entries above its bins; the thread whose bins hold
//      rank K (1-based, from the largest key) hands its B bins to the lanes
//      of its wave, whose scan finds the boundary key t and the number q of
//      entries equal to t that are kept, for K = K1 and K = K2;
//   3. per round, the counts of key > t1, key == t1, key > t2, key == t2
//      (the lanes' exclusive counts stay in registers for step 4);
//   4. the counts' exclusive scans over the rounds (one wave for RW = 16,
//      read from LDS after a barrier; each wave for RW = 4, where a barrier
//      costs more than the scan); each wave places the entries of its
//      rounds that meet a needed range (rank_group step 6).
// Entries past n are loaded as key 0 and not counted in the histogram; they
// come after every real entry, so a boundary at key 0 keeps real zeros
// first (the quota q counts real entries only). Returns the ranking waves'
// barrier count (RW = 4).
template <int RW>
__device__ __attribute__((noinline)) uint32_t rank_all(const uint16_t* __restrict__ x, int n,
                                                       uint32_t K1, uint32_t K2, int list_off,
                                                       uint32_t epoch, uint32_t* status) {
  x = uniform_ptr(x);
  n = (int)uniform((uint32_t)n);
  K1 = uniform(K1);
  K2 = uniform(K2);
  list_off = (int)uniform((uint32_t)list_off);
  epoch = uniform(epoch);
  status = uniform_ptr(status);
  LayerShared& sm = g_sm;
  uint16_t* list = sm.lists + list_off;
  uint32_t* hist = reinterpret_cast<uint32_t*>(sm.keys);  // bins 2 i and 2 i + 1 in word i
  constexpr int kThreads = 64 * RW;
  const int rt = (int)threadIdx.x - (kWaves - RW) * 64;  // ranking thread
  const int lane = rt & 63;
  const int rw = (int)uniform((uint32_t)(rt >> 6));
  constexpr int kPer = 4;                                     // rounds per wave
  constexpr int kBins = kLayerMaxN / kThreads;                // bins per ranking thread
  constexpr int kWords = kBins / 2;
  constexpr int kBinsPerLane = kBins > 64 ? kBins / 64 : 1;  // holder search
  static_assert(kBins % 8 == 0 && kBinsPerLane <= 2, "whole 16-byte reads, two bins per lane");
  const int R = (n + kRankRound - 1) / kRankRound;
  const int Rfull = n / kRankRound;
  auto sync = [&] {
    if constexpr (RW == kWaves)
      lds_barrier();
    else
      rank_sync<RW>(epoch, status);
  };

  // 1. keys (loads in flight while the histogram is cleared)
  const __amdgpu_buffer_rsrc_t rs = tier_rsrc(reinterpret_cast<const uint8_t*>(x), 2u * n);
  uint4 kv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = rw + RW * i;
    kv[i] = make_uint4(0u, 0u, 0u, 0u);
    if (r < Rfull) {
      kv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, 2u * (uint32_t)(r * kRankRound + 8 * lane), 0, 0));
    } else if (r < R) {
      // the round that holds the end of x, entry by entry: the buffer's
      // range ends at x's end and a load past it returns 0, the key of the
      // padding, so all eight loads go out at once with no branch between
      // them (branches made the compiler wait for each pair in turn)
      const uint32_t e = (uint32_t)(r * kRankRound + 8 * lane);
      uint32_t hw[8];
#pragma unroll
      for (int h = 0; h < 8; ++h)
        hw[h] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * (e + (uint32_t)h), 0, 0);
      kv[i] = make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                         hw[6] | (hw[7] << 16));
    }
  }
#pragma unroll
  for (int j = 0; j < kWords / 4; ++j)
    reinterpret_cast<uint4*>(hist)[rt + kThreads * j] = make_uint4(0u, 0u, 0u, 0u);
  if (rt == 0)
    *reinterpret_cast<uint4*>(&sm.rsel[0]) = make_uint4(kAboveAll, 0u, kAboveAll, 0u);
  sync();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = rw + RW * i;
    if (r < R) {
      const uint4 v = make_uint4(kv[i].x & 0x7FFF7FFFu, kv[i].y & 0x7FFF7FFFu,
                                 kv[i].z & 0x7FFF7FFFu, kv[i].w & 0x7FFF7FFFu);
      kv[i] = v;
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      if (r < Rfull) {  // wave-uniform
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t k = (w4[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
          atomicAdd(&hist[k >> 1], 1u << ((k & 1u) << 4));
        }
      } else {
        const int lim = n - (r * kRankRound + 8 * lane);  // real entries of the lane
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t k = (w4[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
          if (h < lim) atomicAdd(&hist[k >> 1], 1u << ((k & 1u) << 4));
        }
      }
    }
  }
  sync();

  // 2. boundary keys and quotas
  {
    const uint4* hp = reinterpret_cast<const uint4*>(hist) + (kWords / 4) * rt;
    uint32_t sum = 0u;  // packed: no half reaches 2^16
#pragma unroll
    for (int j = 0; j < kWords / 4; ++j) {
      const uint4 v = hp[j];
      sum += v.x + v.y + v.z + v.w;
    }
    const uint32_t tot = (sum & 0xFFFFu) + (sum >> 16);
    const uint32_t incl = wave_incl_scan(tot);
    const uint32_t wsum = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (lane == 0) sm.wtot[rw] = wsum;
    sync();
    uint32_t above = wsum - incl;  // entries in the bins of higher lanes of this wave
#pragma unroll
    for (int j = 0; j < RW; ++j) above += j > rw ? sm.wtot[j] : 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t K = c == 0 ? K1 : K2;
      const uint64_t m = __ballot(K > 0u && above < K && K <= above + tot);
      if (m != 0) {  // wave-uniform: this wave holds rank K
        const int L = (int)__builtin_ctzll(m);
        const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
        const int b_top = kBins * (64 * rw + L) + kBins - 1;  // the holder's highest bin
        // lane l takes bins b_top - kBinsPerLane l - (0 .. kBinsPerLane - 1)
        const bool act = lane * kBinsPerLane < kBins;
        const int b0 = b_top - kBinsPerLane * lane;
        const uint32_t c0 = act ? (uint32_t)sm.keys[b0] : 0u;
        const uint32_t c1 = act && kBinsPerLane == 2 ? (uint32_t)sm.keys[b0 - 1] : 0u;
        const uint32_t cnt = c0 + c1;
        const uint32_t ci = ab + wave_incl_scan(cnt);  // through this lane's bins
        const uint32_t cb = ci - cnt;                   // before them
        const uint64_t f = __ballot(act && cb < K && K <= ci);
        const int J = (int)__builtin_ctzll(f);
        if (lane == J) {
          const bool first = K <= cb + c0;  // in the lane's higher bin
          sm.rsel[2 * c] = (uint32_t)(first ? b0 : b0 - 1);
          sm.rsel[2 * c + 1] = first ? K - cb : K - cb - c0;
        }
      }
    }
  }
  sync();
  const uint4 sel = *reinterpret_cast<const uint4*>(&sm.rsel[0]);
  const uint32_t t1 = uniform(sel.x), q1 = uniform(sel.y), t2 = uniform(sel.z),
                 q2 = uniform(sel.w);

  // 3. per-round counts
  uint32_t x1[kPer], x2[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = rw + RW * i;
    x1[i] = x2[i] = 0u;
    if (r < R) {
      uint32_t c1, c2;
      lane_counts(kv[i], t1, t2, c1, c2);
      const uint32_t i1 = wave_incl_scan(c1), i2 = wave_incl_scan(c2);
      x1[i] = i1 - c1;
      x2[i] = i2 - c2;
      if (lane == 63)
        *reinterpret_cast<uint4*>(&sm.rtot[r][0]) =
            make_uint4(i1 & 0xFFFFu, i1 >> 16, i2 & 0xFFFFu, i2 >> 16);
    }
  }
  sync();

  // 4. exclusive counts before each round (lane l: round l); the counts
  // through round r are those before round r + 1, after the last the totals
  uint32_t ex[4] = {0u, 0u, 0u, 0u}, inc[4] = {0u, 0u, 0u, 0u};
  if (RW != kWaves || rw == 0) {
    const uint4 u = lane < R ? *reinterpret_cast<const uint4*>(&sm.rtot[lane][0])
                             : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t own[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      inc[q] = wave_incl_scan(own[q]);
      ex[q] = inc[q] - own[q];
    }
    if (RW == kWaves) {  // shared through LDS
      if (lane < R)
        *reinterpret_cast<uint4*>(&sm.rtot[lane][0]) = make_uint4(ex[0], ex[1], ex[2], ex[3]);
      if (lane == 63)
        *reinterpret_cast<uint4*>(&sm.rsum[0]) = make_uint4(inc[0], inc[1], inc[2], inc[3]);
    }
  }
  if constexpr (RW == kWaves) lds_barrier();
  const Placement P = load_placement(K1, t1, q1, t2, q2);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = rw + RW * i;
    if (r >= R) break;  // wave-uniform
    uint32_t G1, E1, G2, E2, G1e, E1e, G2e, E2e;
    if constexpr (RW == kWaves) {
      const uint4 e = *reinterpret_cast<const uint4*>(&sm.rtot[r][0]);
      const uint4 f = r + 1 < R ? *reinterpret_cast<const uint4*>(&sm.rtot[r + 1][0])
                                : *reinterpret_cast<const uint4*>(&sm.rsum[0]);
      G1 = uniform(e.x); E1 = uniform(e.y); G2 = uniform(e.z); E2 = uniform(e.w);
      G1e = uniform(f.x); E1e = uniform(f.y); G2e = uniform(f.z); E2e = uniform(f.w);
    } else {
      G1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[0], r));
      E1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[1], r));
      G2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[2], r));
      E2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[3], r));
      G1e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[0], r));
      E1e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[1], r));
      G2e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[2], r));
      E2e = uniform((uint32_t)__builtin_amdgcn_readlane((int)inc[3], r));
    }
    if (!round_needed(P, G1, E1, G2, E2, G1e, E1e, G2e, E2e)) continue;
    place_round(P, list, kv[i], (uint32_t)(r * kRankRound + 8 * lane), x1[i], x2[i], G1, E1, G2,
                E2);
  }
  if constexpr (RW != kWaves) {
    // the ranking waves' next use of the shared arrays comes after this
    // barrier (the lists are complete for the ready flag)
    sync();
  }
  return epoch;
}

// Whether group g runs in the launch's second phase: down, when its input
// is the a this launch's gate/up writes.
__device__ __forceinline__ bool late_group(const LayerArgs& A, int g) {
  return g == SPAX_GROUP_DOWN && A.down_waits;
}

// The positions of group g that workgroup w reads (its segments' ranges,
// two intervals per tier: a workgroup meets at most two partial tiles of a
// group, and a third tile makes the whole list needed), the positions it
// stores to the caller's lists (those of its segment of tile 0: tile 0's
// segments cover every position once) and the caller's list pointers, into
// LDS for the ranking.
__device__ __forceinline__ void set_need(const LayerArgs& A, int g, uint32_t w) {
  const LayerGroupArgs& gr = A.g[g];
  uint32_t f[4] = {0u, 0u, 0u, 0u}, a[4] = {0u, 0u, 0u, 0u}, o[4] = {0u, 0u, 0u, 0u};
  int cnt = 0;
  layer_group_segs(A, g, w, [&](const LayerSeg& s) {
    if (s.t == 0) {
      o[0] = (uint32_t)s.f0;
      o[1] = (uint32_t)s.f1;
      o[2] = (uint32_t)s.a0;
      o[3] = (uint32_t)s.a1;
    }
    const int i = cnt < 2 ? cnt : 1;
    f[2 * i] = (uint32_t)s.f0;
    f[2 * i + 1] = (uint32_t)s.f1;
    a[2 * i] = (uint32_t)s.a0;
    a[2 * i + 1] = (uint32_t)s.a1;
    ++cnt;
  });
  if (cnt > 2) {
    f[0] = 0u; f[1] = (uint32_t)gr.k_full;
    a[0] = 0u; a[1] = (uint32_t)gr.k_approx;
  }
  *reinterpret_cast<uint4*>(&g_sm.need[0]) = make_uint4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<uint4*>(&g_sm.need[4]) = make_uint4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<uint4*>(&g_sm.own[0]) = make_uint4(o[0], o[1], o[2], o[3]);
  g_sm.rank_out[0] = reinterpret_cast<uint64_t>(gr.out_full);
  g_sm.rank_out[1] = reinterpret_cast<uint64_t>(gr.out_approx);
}

// The first group in processing order that workgroup w ranks, or -1.
__device__ __forceinline__ int first_ranked(const LayerArgs& A, uint32_t w) {
  // (unrolled: every group's fields sit at fixed offsets of the arguments)
#pragma unroll
  for (int oi = 0; oi < 4; ++oi) {
    const int g = layer_order(oi);
    if (layer_meets(A, g, w) && A.g[g].k_full + A.g[g].k_approx > 0 && !late_group(A, g))
      return g;
  }
  return -1;
}

// Waits (bounded) until every gate/up tile has written its a.
__device__ __forceinline__ void wait_gate_up(const LayerArgs& A) {
  uint32_t* status = A.sync + 2;
  const uint32_t need = (uint32_t)A.g[SPAX_GROUP_GATE_UP].tiles;
  for (uint32_t k = 0;
       __hip_atomic_load(&A.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need; ++k) {
    if (k >= kSpinGlobal) {
      if ((threadIdx.x & 63) == 0) set_status(status, kStatusGlobalWait);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // acquire at agent scope: the caches are invalidated, so plain loads of a
  // by any wave of the workgroup (after its barrier) see the gate/up stores
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Ranking waves: rank each further group of the first phase that the
// workgroup meets, in processing order (the first was ranked by the whole
// workgroup).
__device__ __forceinline__ void rank_role(const LayerArgs& A, int first, uint32_t epoch) {
  __builtin_amdgcn_s_setprio(3);
  uint32_t* status = A.sync + 2;
  const uint32_t w = blockIdx.x;
  const int rt = (int)threadIdx.x - (kLayerStreamWaves + 1) * 64;
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    if (g == first || late_group(A, g) || !layer_meets(A, g, w)) continue;
    const LayerGroupArgs& gr = A.g[g];
    const uint32_t K1 = (uint32_t)gr.k_full, K2 = (uint32_t)(gr.k_full + gr.k_approx);
    if (K2 == 0u) continue;  // no lists: the group's segments are empty
    if (rt == 0) set_need(A, g, w);
    // (inputs past four rounds per ranking wave: the LDS-keys ranking)
    if (gr.n <= 4 * kRankRound * kLayerRankWaves)
      epoch = rank_all<kLayerRankWaves>(gr.x, gr.n, K1, K2, gr.list_off, epoch, status);
    else
      epoch = rank_group<kLayerRankWaves>(gr.x, gr.n, K1, K2, gr.list_off, epoch, status);
    if (rt == 0) lds_signal_store(&g_sm.ready[g], 1u);
  }
}

// ---- streaming ---------------------------------------------------------
// In each phase the streaming waves split between the two tiers once, in
// proportion to the tiers' streaming cost over the workgroup's segments of
// the phase; in every segment a wave takes an equal share of its tier's
// list positions. A wave streams all its shares as one sequence through a
// ring of loads in registers: the load for ring slot u is issued as soon as
// slot u's previous load has been added, across segment boundaries, so the
// ring never drains between segments. The rings are short (3 KB of fp16
// columns in flight per wave): with more requests in flight the chip's
// scattered 1 KB reads got slower, not faster, and with 2 the ring drained
// (measured on 7B layers). When a segment's last load has been
// added, the wave hands its fp32 partial of the tile's 512 rows to the
// reduction wave through LDS (two slot sets, so a wave can run one segment
// ahead) and starts the next sum. A share with no positions still costs one
// load, with a zero factor, so every wave hands over every segment.
// Column indices come from the LDS list: lane l holds the entry of position
// 64 b + l of the share's batch b that the issue pointer is in.

// Streaming cost of one column's 512-row tile per format: its bytes,
// weighted by how much slower a code wave streams a byte than an fp16 wave
// (more vector work, and two small loads per code load; measured on 7B
// layers).
__host__ __device__ constexpr uint32_t form_tile_cost(int fmt) {
  return fmt == kFp16 ? 1026u : fmt == kInt4 ? 426u : 800u;
}

// Per-format streaming: fp16 columns load one column per load, lane l
// reading rows 8 l .. 8 l + 7 of the tile (16 bytes). Code tiers load four
// columns per load: lane (q, i) = (lane / 16, lane mod 16) reads rows
// 32 i .. 32 i + 31 of the load's q-th column (16 bytes of int4 codes, 8 of
// 2-bit codes), so one load moves as many bytes as an fp16 column; the
// lane's rows lie in one 128-row group g = i / 4, and it loads its own x_j
// and scale s_{j,g} with the codes.
template <int FMT>
struct Form;
template <>
struct Form<kFp16> {
  using V = uint4;
  static constexpr int kRing = 3;
  static constexpr int kPos = 1;  // list positions per load
};
template <>
struct Form<kInt4> {
  using V = uint4;
  static constexpr int kRing = 4;
  static constexpr int kPos = 4;
  static constexpr uint32_t kLaneBytes = 16;
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
  }
  static __device__ __forceinline__ uint32_t piece(const V& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};
template <>
struct Form<kInt2> {
  using V = uint2;
  static constexpr int kRing = 6;
  static constexpr int kPos = 4;
  static constexpr uint32_t kLaneBytes = 8;
  static __device__ __forceinline__ V load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0));
  }
  static __device__ __forceinline__ uint32_t piece(const V& v, int k) {
    const uint32_t w = k < 2 ? v.x : v.y;
    return (k & 1) ? (w >> 16) : (w & 0xFFFFu);
  }
};
template <>
struct Form<kSign2> : Form<kInt2> {};

// Workgroup w's segments of one phase into the LDS table, in processing
// order, by one wave: lane i builds entries i, i + 64, ...
__device__ __forceinline__ void build_segtab(const LayerArgs& A, uint32_t w, bool late) {
  const int lane = (int)threadIdx.x & 63;
  uint32_t base = 0u;
  // unrolled over the groups: their fields sit at fixed offsets of the
  // arguments, and the four range computations are independent
#pragma unroll
  for (int oi = 0; oi < 4; ++oi) {
    const int g = layer_order(oi);
    uint32_t t0, step, t_end, u0, u1;
    if (late_group(A, g) != late || !layer_group_range(A, g, w, t0, step, t_end, u0, u1))
      continue;
    const uint32_t cnt = step == 1u ? t_end - t0 : (t_end - t0 + step - 1u) / step;
    // (the host keeps every phase within the table)
    for (uint32_t i = (uint32_t)lane; i < cnt && base + i < (uint32_t)kLayerSegTab; i += 64u) {
      const LayerSeg sg = layer_make_seg(A, g, w, t0 + i * step, u0, u1);
      g_sm.segtab[base + i] = make_uint4((uint32_t)sg.g | ((uint32_t)sg.t << 8),
                                         (uint32_t)sg.f0 | ((uint32_t)sg.f1 << 16),
                                         (uint32_t)sg.a0 | ((uint32_t)sg.a1 << 16), 0u);
    }
    base += cnt;
  }
  if (lane == 0) g_sm.nseg = min(base, (uint32_t)kLayerSegTab);
}

// Entry i of the segment table (wave-uniform).
__device__ __forceinline__ LayerSeg table_seg(uint32_t i) {
  const uint4 e = g_sm.segtab[i];
  LayerSeg s;
  s.g = (int)uniform(e.x & 0xFFu);
  s.t = (int)uniform(e.x >> 8);
  s.f0 = (int)uniform(e.y & 0xFFFFu);
  s.f1 = (int)uniform(e.y >> 16);
  s.a0 = (int)uniform(e.z & 0xFFFFu);
  s.a1 = (int)uniform(e.z >> 16);
  s.w_lo = s.w_hi = -1;
  return s;
}

// floor(a / b) for a < 2^24 and 1 <= b <= 16, with b's reciprocal rb.
__device__ __forceinline__ int small_div(int a, int b, float rb) {
  int q = (int)((float)a * rb);
  q += (q + 1) * b <= a ? 1 : 0;
  q -= q * b > a ? 1 : 0;
  return q;
}

// A segment's share of one tier, as the issue side of a streaming wave sees
// it (all wave-uniform but the per-lane offsets).
struct Share {
  const uint16_t* list;   // the share's first list entry (LDS)
  int n;                  // positions
  int loads;              // max(1, ceil(n / positions per load))
  __amdgpu_buffer_rsrc_t rs, xr, sr;
  uint32_t stride, sstride;
  uint32_t off;           // fp16: the lane's byte offset in a column
  uint32_t sg;            // codes: the lane's scale index in a column (the sign
                          // code: its matrix's (s0, s1) pair)
};

// The share of tier `full` of segment s for wave wi of nw on that tier.
template <int FMT>
__device__ __forceinline__ Share make_share(const LayerArgs& A, const LayerSeg& s, bool full,
                                            int wi, int nw, float rnw) {
  const LayerGroupArgs& gr = A.g[s.g];
  const int lane = (int)threadIdx.x & 63;
  const int p0 = full ? s.f0 : s.a0, np = full ? s.f1 - s.f0 : s.a1 - s.a0;
  const int lo = p0 + small_div(np * wi, nw, rnw), hi = p0 + small_div(np * (wi + 1), nw, rnw);
  Share h;
  h.list = g_sm.lists + gr.list_off + (full ? 0 : gr.k_full) + lo;
  h.n = hi - lo;
  h.loads = max(1, (h.n + Form<FMT>::kPos - 1) / Form<FMT>::kPos);
  h.rs = tier_rsrc(full ? gr.full_base : gr.approx_base, full ? gr.full_bytes : gr.approx_bytes);
  h.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(gr.x), (short)0, 0x7FFFFFFF,
                                           0x00020000);
  const uint16_t* sc = full ? gr.full_scales : gr.approx_scales;
  h.sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc), (short)0, 0x7FFFFFFF,
                                           0x00020000);
  h.stride = (uint32_t)(full ? gr.full_stride : gr.approx_stride);
  h.sstride = (uint32_t)(full ? gr.full_sstride : gr.approx_sstride);
  const int row0 = s.t * kTileRows;
  if constexpr (FMT == kFp16) {
    // lanes past the last row of a ragged tile read lane 0's rows; their
    // sums are never stored
    const int ld = row0 + 8 * lane < gr.rows ? lane : 0;
    h.off = 2u * (uint32_t)(row0 + 8 * ld);
    h.sg = 0u;
  } else {
    const int li = row0 + 32 * (lane & 15) < gr.rows ? (lane & 15) : 0;
    h.off = (uint32_t)(row0 + 32 * li) / 32u * Form<FMT>::kLaneBytes;
    if constexpr (FMT == kSign2) {
      // the matrix of the lane's rows in a stored column that holds several
      // (each coded as its own column): GLU gate / up by 128-row block
      // parity, or the stacked segment of the tile
      const int seg = gr.approx_seg < 0   ? ((row0 + 32 * li) >> 7) & 1
                      : gr.approx_seg > 0 ? row0 / gr.approx_seg
                                          : 0;
      h.sg = (uint32_t)seg;
    } else {
      h.sg = (uint32_t)(row0 / kGroup + li / 4);
    }
  }
  return h;
}

// Hands partial p (the 8 rows of row block `block`) of the wave's segment k
// to the reduction wave.
__device__ __forceinline__ void hand_over(int sw, uint32_t k, int block, const float (&p)[8],
                                          uint32_t* status) {
  LayerShared& sm = g_sm;
  // slot set k & 1 was last read for segment k - 2
  if (k >= 2u) wait_lds_ge(&sm.seg_free, k - 1u, status);
  float4* dst = reinterpret_cast<float4*>(&sm.slot[k & 1u][sw][8 * block]);
  dst[0] = make_float4(p[0], p[1], p[2], p[3]);
  dst[1] = make_float4(p[4], p[5], p[6], p[7]);
  if ((threadIdx.x & 63) == 0) lds_signal_add(&sm.seg_arrive[k & 1u], 1u);
}

// Wave wi of the nw streaming waves on tier `full` (format FMT) of one
// phase: every segment's share, as one ring sequence.
template <int FMT>
__device__ __forceinline__ void stream_seq(const LayerArgs& A, bool late, bool full, int wi,
                                           int nw, int sw, uint32_t& k) {
  using Fm = Form<FMT>;
  constexpr int R = Fm::kRing;
  uint32_t* status = A.sync + 2;
  const int lane = (int)threadIdx.x & 63;
  const float rnw = 1.0f / (float)nw;
  const uint32_t nseg = uniform(g_sm.nseg);
  // loads of the whole sequence
  int L = 0;
  for (uint32_t i = 0; i < nseg; ++i) {
    const LayerSeg s = table_seg(i);
    const int np = full ? s.f1 - s.f0 : s.a1 - s.a0;
    const int n = small_div(np * (wi + 1), nw, rnw) - small_div(np * wi, nw, rnw);
    L += max(1, (n + Fm::kPos - 1) / Fm::kPos);
  }
  if (L == 0) return;
  uint32_t si = 0u;  // next table entry
  Share sh;
  sh.loads = 0;
  int j = 0;         // next load of the current share
  int colv = 0;      // list entries of the issue pointer's batch
  uint32_t ends = 0; // ring slots holding the last load of a share
  // fp16: 8 sums; codes: 32 (rows 32 i + 8 k + r) and the offset sum
  constexpr int kAcc = FMT == kFp16 ? 1 : 4;
  float acc[kAcc][8];
#pragma unroll
  for (int q = 0; q < kAcc; ++q)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[q][r] = 0.0f;
  float corr = 0.0f;
  typename Fm::V d[R];
  uint32_t xs[R], ss[R];
  const uint32_t kM = [] {
    uint32_t m = FMT == kFp16 ? 0u : Tier<FMT>::kMask;
    asm volatile("" : "+v"(m));  // a VGPR, not a literal
    return m;
  }();

  // issue side: the next load into ring slot u (past the sequence, the last
  // load again; it is never added)
  auto issue = [&](int u) {
    bool redo = false;
    if (j == sh.loads) {
      if (si < nseg) {
        const LayerSeg seg = table_seg(si++);
        sh = make_share<FMT>(A, seg, full, wi, nw, rnw);
        j = 0;
        if (sh.n > 0) {
          wait_lds_ge(&g_sm.ready[seg.g], 1u, status);
          colv = (int)sh.list[min(lane, sh.n - 1)];
        }
      } else {
        redo = true;
      }
    }
    const int jj = redo ? sh.loads - 1 : j;
    if (!redo) {
      if ((jj * Fm::kPos & 63) == 0 && jj > 0)
        colv = (int)sh.list[min(jj * Fm::kPos + lane, sh.n - 1)];  // the next batch
      ends = (ends & ~(1u << u)) | ((jj == sh.loads - 1 ? 1u : 0u) << u);
      ++j;
    }
    if constexpr (FMT == kFp16) {
      const bool live = jj < sh.n;  // wave-uniform
      const uint32_t col = live ? (uint32_t)__builtin_amdgcn_readlane(colv, jj & 63) : 0u;
      d[u] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(sh.rs, sh.off, col * sh.stride, 0));
      xs[u] = live ? __builtin_amdgcn_raw_buffer_load_b16(sh.xr, 0u, 2u * col, 0) : 0u;
    } else {
      const int q = lane >> 4;
      const int pos = 4 * jj + q;
      const bool live = pos < sh.n;
      const uint32_t col =
          (uint32_t)__builtin_amdgcn_ds_bpermute((min(pos, max(sh.n - 1, 0)) & 63) << 2, colv);
      const uint32_t c = sh.n > 0 ? col : 0u;
      d[u] = Fm::load(sh.rs, c * sh.stride + sh.off);
      xs[u] = live ? __builtin_amdgcn_raw_buffer_load_b16(sh.xr, 2u * c, 0, 0) : 0u;
      if constexpr (FMT == kSign2)
        ss[u] = __builtin_amdgcn_raw_buffer_load_b32(sh.sr, 2u * (c * sh.sstride + 2u * sh.sg), 0,
                                                     0);
      else
        ss[u] = __builtin_amdgcn_raw_buffer_load_b16(sh.sr, 2u * (c * sh.sstride + sh.sg), 0, 0);
    }
  };

  // consume side: adds ring slot u; at a share's last load hands the
  // segment's partial over
  auto consume = [&](int u) {
    if constexpr (FMT == kFp16) {
      const float f = h2f(xs[u]);
      const uint4 v = d[u];
      acc[0][0] = fmaf(h2f(v.x & 0xFFFFu), f, acc[0][0]);
      acc[0][1] = fmaf(h2f(v.x >> 16), f, acc[0][1]);
      acc[0][2] = fmaf(h2f(v.y & 0xFFFFu), f, acc[0][2]);
      acc[0][3] = fmaf(h2f(v.y >> 16), f, acc[0][3]);
      acc[0][4] = fmaf(h2f(v.z & 0xFFFFu), f, acc[0][4]);
      acc[0][5] = fmaf(h2f(v.z >> 16), f, acc[0][5]);
      acc[0][6] = fmaf(h2f(v.w & 0xFFFFu), f, acc[0][6]);
      acc[0][7] = fmaf(h2f(v.w >> 16), f, acc[0][7]);
    } else if constexpr (FMT == kSign2) {
      const float xj = h2f(xs[u]);
      const float fa = xj * h2f(ss[u] & 0xFFFFu), fb = xj * h2f(ss[u] >> 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) Tier<FMT>::fma2(acc[q], Fm::piece(d[u], q), fa, fb, kM);
    } else {
      const float f = h2f(xs[u]) * h2f(ss[u]) * Tier<FMT>::kScale;
      if constexpr (FMT == kInt2) {
        // one 32-bit word holds rows 16 w .. 16 w + 15 (row k in bits 2k,
        // 2k + 1): one shift puts rows k and k + 8 into bits 8..9 of the two
        // halves, so each pair costs a shift and an and-or (fp16 1 + u / 4)
        const uint32_t dw[2] = {d[u].x, d[u].y};
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t sh = k <= 4 ? dw[w] << (8 - 2 * k) : dw[w] >> (2 * k - 8);
            const uint32_t p = (sh & kM) | 0x3C003C00u;
            acc[2 * w][k] = fmaf(h2f(p & 0xFFFFu), f, acc[2 * w][k]);
            acc[2 * w + 1][k] = fmaf(h2f(p >> 16), f, acc[2 * w + 1][k]);
          }
      } else {
        float unused = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) Tier<FMT>::fma(acc[q], unused, Fm::piece(d[u], q), f, kM);
      }
      corr = fmaf(FMT == kInt4 ? 1.5f : 1.375f, f, corr);
    }
    if ((ends >> u) & 1u) {  // wave-uniform
      float p[8];
      int block = lane;
      if constexpr (FMT == kFp16) {
#pragma unroll
        for (int r = 0; r < 8; ++r) p[r] = acc[0][r];
      } else {
        // the four quarters' sums, added across lanes: q with q ^ 2 (lanes
        // q < 2 keep row pieces 0, 1), then q with q ^ 1 (even q keep the
        // first piece); lane (q, i) ends with rows 32 i + 8 q .. + 7
        if constexpr (FMT != kSign2) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[q][r] -= corr;
        }
        const int q = lane >> 4;
        const bool lo = q < 2, ev = (q & 1) == 0;
        float h[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float keep = lo ? acc[kk][r] : acc[kk + 2][r];
            const float send = lo ? acc[kk + 2][r] : acc[kk][r];
            h[kk][r] = keep + __shfl_xor(send, 32, 64);
          }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float keep = ev ? h[0][r] : h[1][r];
          const float send = ev ? h[1][r] : h[0][r];
          p[r] = keep + __shfl_xor(send, 16, 64);
        }
        block = 4 * (lane & 15) + q;
      }
      hand_over(sw, k, block, p, status);
      ++k;
#pragma unroll
      for (int q = 0; q < kAcc; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[q][r] = 0.0f;
      corr = 0.0f;
    }
  };

#pragma unroll
  for (int u = 0; u < R; ++u) issue(u);
  for (int c0 = 0; c0 < L; c0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (c0 + u < L) consume(u);  // wave-uniform
      issue(u);
    }
  }
}

// Streaming waves of one phase: the split between the tiers, then the wave's
// sequence.
template <int FF, int AF>
__device__ __forceinline__ void stream_role(const LayerArgs& A, int sw, bool late, uint32_t& k) {
  const uint32_t nseg = uniform(g_sm.nseg);
  uint64_t cf = 0, ca = 0;
  for (uint32_t i = 0; i < nseg; ++i) {
    const LayerSeg s = table_seg(i);
    cf += (uint64_t)(s.f1 - s.f0) * form_tile_cost(FF);
    ca += (uint64_t)(s.a1 - s.a0) * form_tile_cost(AF);
  }
  int wf = kNS;
  if (AF != kNone && ca > 0) {
    wf = cf == 0 ? 0 : (int)((2u * kNS * cf + cf + ca) / (2u * (cf + ca)));
    if (cf > 0) wf = min(max(wf, 1), kNS - 1);
  }
  if (sw < wf)
    stream_seq<FF>(A, late, true, sw, wf, sw, k);
  else if constexpr (AF != kNone)
    stream_seq<AF>(A, late, false, sw - wf, kNS - wf, sw, k);
}

// Output of one tile: fp16 y, or for gate/up a = silu(g) * u from the fp16
// g and u (lane l holds gate rows, lane l + 16 the matching up rows), then
// the tile is counted in for down's ranking.
__device__ __forceinline__ void finish_tile(const LayerArgs& A, const LayerSeg& s,
                                            const float (&p)[8], int lane) {
  const LayerGroupArgs& gr = A.g[s.g];
  const int r0 = s.t * kTileRows + 8 * lane;
  if (s.g != SPAX_GROUP_GATE_UP) {
    if (r0 < gr.rows) {
      uint4 o;
      o.x = (uint32_t)f2h(p[0]) | ((uint32_t)f2h(p[1]) << 16);
      o.y = (uint32_t)f2h(p[2]) | ((uint32_t)f2h(p[3]) << 16);
      o.z = (uint32_t)f2h(p[4]) | ((uint32_t)f2h(p[5]) << 16);
      o.w = (uint32_t)f2h(p[6]) | ((uint32_t)f2h(p[7]) << 16);
      *reinterpret_cast<uint4*>(gr.y + r0) = o;
    }
    return;
  }
  float up[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) up[r] = __shfl_down(p[r], 16, 64);
  if ((lane & 16) == 0 && r0 < gr.rows) {
    const int gi = s.t * 256 + (lane >> 5) * 128 + 8 * (lane & 15);
    uint32_t av[4], gv[4], uv[4];
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
      uint32_t ab[2], gb[2], ub[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        gb[h] = f2h(p[r + h]);
        ub[h] = f2h(up[r + h]);
        const float g = h2f(gb[h]), u = h2f(ub[h]);
        ab[h] = f2h(g / (1.0f + expf(-g)) * u);
      }
      av[r / 2] = ab[0] | (ab[1] << 16);
      gv[r / 2] = gb[0] | (gb[1] << 16);
      uv[r / 2] = ub[0] | (ub[1] << 16);
    }
    // a is read by down's ranking in other workgroups: a coherent store
    const __amdgpu_buffer_rsrc_t ra =
        tier_rsrc(reinterpret_cast<const uint8_t*>(A.glu_a), (uint32_t)gr.rows);
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t,
                           make_uint4(av[0], av[1], av[2], av[3])),
        ra, 2u * gi, 0, kCoherent);
    if (A.glu_g) *reinterpret_cast<uint4*>(A.glu_g + gi) = make_uint4(gv[0], gv[1], gv[2], gv[3]);
    if (A.glu_u) *reinterpret_cast<uint4*>(A.glu_u + gi) = make_uint4(uv[0], uv[1], uv[2], uv[3]);
  }
  if (A.down_waits) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores of a are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0)
      __hip_atomic_fetch_add(&A.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The final sum of a tile with many contributors (down in the second
// phase: about 32 per tile for a 4096-row down on 256 workgroups), shared by
// the last kFinalParts contributors to count in: the one that arrived
// kFinalParts - 1 - p before the last waits (bounded) until every
// contributor has counted in, then adds row slice p of the tile over all
// contributors' partials, in workgroup order, and writes its y. One CU
// reading every partial of the tile (64 KB) takes several times as long as
// eight CUs reading an eighth each (measured on the 7B layer: 6.30 against
// 6.66 ms per 32-layer step; four parts 6.32). The last of the kFinalParts
// to finish clears the tile's counts.
__device__ __forceinline__ void split_final(const LayerArgs& A, const LayerSeg& s,
                                            __amdgpu_buffer_rsrc_t rp, int base_slot,
                                            uint32_t* ctr, uint32_t old, uint32_t nc, int lane,
                                            uint32_t* status) {
  if (old + kFinalParts < nc) return;  // not one of the last kFinalParts
  const uint32_t part = old - (nc - kFinalParts);
  for (uint32_t it = 0; old + 1u < nc &&
                        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nc;
       ++it) {
    if (it >= kSpinGlobal) {
      if (lane == 0) set_status(status, kStatusGlobalWait);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // lane l: row l of the slice; up to 32 contributors' loads in flight
  const int rr = (int)part * kPartRows + lane;
  const uint32_t lo = (uint32_t)(4 * rr);
  float q0 = 0.0f;
  for (int c0 = s.w_lo; c0 <= s.w_hi; c0 += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int cc = min(c0 + u, s.w_hi);
      const uint32_t o = (uint32_t)((base_slot + cc) * kTileRows * 4) + lo;
      v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, o, 0, kCoherent));
    }
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (c0 + u <= s.w_hi) q0 += v[u];
  }
  const LayerGroupArgs& gr = A.g[s.g];
  const int r = s.t * kTileRows + rr;
  if (r < gr.rows) gr.y[r] = f2h(q0);
  // the tile's counts back to zero once every slice's adder has seen them
  // (word g + 4 of the tile's counter block is free: the groups use 0..3)
  if (lane == 0) {
    uint32_t* done = ctr + 4;
    const uint32_t d = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == kFinalParts - 1u) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Reduction wave: per segment, the workgroup's partial of the tile, then the
// cross-workgroup sum by the tile's last contributor.
__device__ __forceinline__ void reduce_role(const LayerArgs& A, uint32_t& k) {
  LayerShared& sm = g_sm;
  __builtin_amdgcn_s_setprio(3);
  uint32_t* status = A.sync + 2;
  const int lane = (int)threadIdx.x & 63;
  const uint32_t w = blockIdx.x;
  const uint32_t nseg = uniform(sm.nseg);
  for (uint32_t si = 0; si < nseg; ++si) {
    {
      LayerSeg s = table_seg(si);
      const int g = s.g;
      wait_lds_ge(&sm.seg_arrive[k & 1u], (uint32_t)kNS * (k / 2u + 1u), status);
      float p[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] = 0.0f;
#pragma unroll
      for (int q = 0; q < kNS; ++q) {
        const float4* src = reinterpret_cast<const float4*>(&sm.slot[k & 1u][q][8 * lane]);
        const float4 u0 = src[0], u1 = src[1];
        p[0] += u0.x; p[1] += u0.y; p[2] += u0.z; p[3] += u0.w;
        p[4] += u1.x; p[5] += u1.y; p[6] += u1.z; p[7] += u1.w;
      }
      ++k;
      if (lane == 0) lds_signal_store(&sm.seg_free, k);
      layer_contributors(A, s);
      if (s.w_lo == s.w_hi) {  // the only contributor
        finish_tile(A, s, p, lane);
        continue;
      }
      const LayerGroupArgs& gr = A.g[g];
      const uint32_t pbytes = (uint32_t)((gr.tiles + gr.n_wg) * kTileRows * 4);
      const __amdgpu_buffer_rsrc_t rp =
          tier_rsrc(reinterpret_cast<const uint8_t*>(gr.partials), pbytes);
      // slot t + i for the workgroup's index i within the group
      const int base_slot = s.t - gr.wg_lo;
      const uint32_t off = (uint32_t)(((base_slot + (int)w) * kTileRows + 8 * lane) * 4);
      using V4 = __attribute__((ext_vector_type(4))) uint32_t;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(V4, make_float4(p[0], p[1], p[2], p[3])), rp, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(V4, make_float4(p[4], p[5], p[6], p[7])), rp, off + 16u, 0,
          kCoherent);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // the partial is stored
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      uint32_t* ctr = gr.counters + s.t * kCountersPerTile;
      uint32_t old = 0u;
      if (lane == 0)
        old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = (uint32_t)__builtin_amdgcn_readlane((int)old, 0);
      const uint32_t nc = (uint32_t)(s.w_hi - s.w_lo + 1);
      if (late_group(A, g) && nc >= 2u * kFinalParts) {
        split_final(A, s, rp, base_slot, ctr, old, nc, lane, status);
        continue;
      }
      if (old != nc - 1u) continue;
      if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      // the last contributor: add every contributor's partial in workgroup
      // order
      float q8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) q8[r] = 0.0f;
      const uint32_t lane_off = (uint32_t)(8 * lane * 4);
      for (int c0 = s.w_lo; c0 <= s.w_hi; c0 += 8) {
        float4 v[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int cc = min(c0 + u, s.w_hi);
          const uint32_t o = (uint32_t)((base_slot + cc) * kTileRows * 4) + lane_off;
          v[u][0] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(rp, o, 0, kCoherent));
          v[u][1] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(rp, o + 16u, 0, kCoherent));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (c0 + u <= s.w_hi) {
            q8[0] += v[u][0].x; q8[1] += v[u][0].y; q8[2] += v[u][0].z; q8[3] += v[u][0].w;
            q8[4] += v[u][1].x; q8[5] += v[u][1].y; q8[6] += v[u][1].z; q8[7] += v[u][1].w;
          }
        }
      }
      finish_tile(A, s, q8, lane);
    }
  }
}

template <int FF, int AF>
__global__ __launch_bounds__(kGemvThreads) void layer_kernel(LayerArgs A) {
  LayerShared& sm = g_sm;
  const int t = (int)threadIdx.x;
  sm.hist[t] = 0u;
  sm.sub[t] = 0u;
  if (t < 4) sm.ready[t] = 0u;
  if (t == 0) {
    sm.rbar = 0u;
    sm.seg_arrive[0] = 0u;
    sm.seg_arrive[1] = 0u;
    sm.seg_free = 0u;
  }
  // the first group the workgroup ranks: every wave ranks it (the streaming
  // waves have nothing to read before it)
  const uint32_t w = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int first = first_ranked(A, w);
  __syncthreads();
  // the first phase's segments (the last wave) and the positions the first
  // ranking places (the wave before it), while the other waves load the
  // first ranking's keys (the placement reads the positions after the
  // ranking's barriers)
  if (wave == kWaves - 1) build_segtab(A, w, false);
  if (first >= 0 && t == (kWaves - 2) * 64) set_need(A, first, w);
  uint32_t epoch = 0u;
  if (first >= 0) {
    const LayerGroupArgs& gr = A.g[first];
    rank_all<kWaves>(gr.x, gr.n, (uint32_t)gr.k_full, (uint32_t)(gr.k_full + gr.k_approx),
                     gr.list_off, 0u, A.sync + 2);
    if (t == 0) sm.ready[first] = 1u;
  }
  lds_barrier();  // the first lists and the segment table are in LDS
  uint32_t k = 0u;  // segments handed over (streaming and reduction waves)
  // phase 0: every group but a late down; phase 1: down, once every gate/up
  // tile has written a (one call site per role keeps the streaming code
  // inlined once)
  for (int phase = 0; phase < 2; ++phase) {
    if (phase == 1) {
      if (!(A.down_waits && layer_meets(A, SPAX_GROUP_DOWN, w))) break;
      // the whole workgroup ranks a: its streaming waves are done with phase 0
      __syncthreads();
      if (wave == 0) {
        wait_gate_up(A);
      } else if (wave == 1) {
        build_segtab(A, w, true);
        if (t == 64) set_need(A, SPAX_GROUP_DOWN, w);
      }
      __syncthreads();
      const LayerGroupArgs& gd = A.g[SPAX_GROUP_DOWN];
      if (gd.k_full + gd.k_approx > 0)
        rank_all<kWaves>(gd.x, gd.n, (uint32_t)gd.k_full, (uint32_t)(gd.k_full + gd.k_approx),
                         gd.list_off, 0u, A.sync + 2);
      if (t == 0) sm.ready[SPAX_GROUP_DOWN] = 1u;
      lds_barrier();
    }
    if (wave < kLayerStreamWaves)
      stream_role<FF, AF>(A, wave, phase == 1, k);
    else if (wave == kLayerReduceWave)
      reduce_role(A, k);
    else if (phase == 0)
      rank_role(A, first, epoch);
  }
  __syncthreads();
  if (t == 0) {
    // the last workgroup to finish resets the launch's counts
    const uint32_t old =
        __hip_atomic_fetch_add(&A.sync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)A.G - 1u) {
      __hip_atomic_store(&A.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&A.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int FF, int AF>
hipError_t launch_pair(const LayerArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((layer_kernel<FF, AF>), dim3((unsigned)a.G), dim3(kGemvThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer(const LayerArgs& a, int32_t full_fmt, int32_t approx_fmt,
                        hipStream_t s) {
  // (layers with an int4 full tier run the per-group launches)
  if (full_fmt == kFp16) {
    if (approx_fmt == kNone) return launch_pair<kFp16, kNone>(a, s);
    if (approx_fmt == kInt4) return launch_pair<kFp16, kInt4>(a, s);
    if (approx_fmt == kInt2) return launch_pair<kFp16, kInt2>(a, s);
    if (approx_fmt == kSign2) return launch_pair<kFp16, kSign2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spax
