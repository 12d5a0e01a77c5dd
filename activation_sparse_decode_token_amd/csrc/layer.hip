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
//   * waves 12..15 rank: for each group the workgroup meets they rank the
//     group's input (two-level radix select on the fp16 magnitude key, lower
//     index first among equal keys) and write the whole ascending F and A
//     lists, with the activations, into LDS. The lists of the next group are
//     ready before the streaming waves reach it, so only the first ranking
//     of a launch is on the critical path.
// Down's input a is complete only when every gate/up tile is: its ranking
// waits for the count of finished gate/up tiles (a bounded wait; gate/up
// runs first on every workgroup, so the count is reached while the q/k/v
// and o columns stream).
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

struct LayerShared {
  uint16_t lists[kLayerListCap];             // every group's F then A lists
  uint16_t keys[kLayerMaxN];                 // ranking: the input's fp16 bits
  float slot[kNS][kTileRows];                // streaming waves' partials
  WaveMeta wm[2][kNS];                       // code factors per tier and wave
  uint32_t hist[256 * kHistCopies];          // ranking: top-level histogram
  uint32_t sub[256 * kHistCopies];           // ranking: the two sub-histograms
  uint32_t rtot[kRankMaxRounds][4];          // ranking: per-round counts
  uint32_t need[8];                          // ranking: positions to place
  uint64_t rank_out[2];                      // ranking: the caller's lists
  uint32_t ready[4];                         // a group's lists are in LDS
  uint32_t rbar;                             // ranking waves' barrier count
  uint32_t seg_arrive;                       // streaming-wave arrivals
  uint32_t seg_free;                         // segments whose slots were read
};
static_assert(sizeof(LayerShared) <= 160 * 1024, "LDS of one workgroup");

// The workgroup's LDS (one instance per launch of any layer kernel).
static __shared__ LayerShared g_sm;

__device__ __forceinline__ uint32_t lds_acquire(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bit) {
  __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the LDS word p reaches v (bounded).
__device__ __forceinline__ void wait_lds_ge(uint32_t* p, uint32_t v, uint32_t* status) {
  for (uint32_t it = 0; lds_acquire(p) < v; ++it) {
    if (it >= kSpinLds) {
      if ((threadIdx.x & 63) == 0) set_status(status, kStatusLdsWait);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
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

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Barrier of the ranking waves: the hardware barrier when every wave of the
// workgroup ranks, else an LDS count (bounded).
template <int RW>
__device__ __forceinline__ void rank_sync(uint32_t& epoch, uint32_t* status) {
  if constexpr (RW == kWaves) {
    __syncthreads();
  } else {
    epoch += RW;
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_fetch_add(&g_sm.rbar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
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

// Ranks x[0, n) on RW waves (the last RW of the workgroup) and places the
// list positions this workgroup needs: the ascending F list (the K1 largest
// |x_j|) at list[0, K1) and the A list (the next K2 - K1) at list[K1, K2),
// one 16-bit column index per entry, each placed entry also stored to the
// caller's lists. The positions needed are g_sm.need: full-tier positions
// [need0, need1) and [need2, need3), approx-tier [need4, need5) and
// [need6, need7). Keys go to LDS once, in rounds of 512 entries (round r on
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
//      (ballots and scalar bit counts);
//   6. their exclusive scans over the rounds give each round's range of
//      list positions; the rounds that meet a needed range are placed in
//      index order, slot by slot (slot h of round r: entries 512 r + 64 h +
//      lane): #F before entry i is gt1 + min(eq1, q1), #(F or A) before it
//      gt2 + min(eq2, q2), counted with ballots and mbcnt.
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

  // 1. keys into LDS (read coherently: down's a is written by this launch),
  // eight rounds of loads in flight per wave; the round that holds the end
  // of x is read entry by entry
  const __amdgpu_buffer_rsrc_t rs = tier_rsrc(reinterpret_cast<const uint8_t*>(x), 2u * n);
  const int Rfull = n / kRankRound;  // rounds entirely inside x
  for (int r0 = rw; r0 < Rfull; r0 += 8 * RW) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(r0 + u * RW, Rfull - 1);
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, 2u * (uint32_t)(r * kRankRound + 8 * lane), 0,
                                           kCoherent));
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
    const int e = Rfull * kRankRound + 8 * lane;
    uint32_t wd[4];
#pragma unroll
    for (int h = 0; h < 8; h += 2) {
      uint32_t lo = 0u, hi = 0u;
      if (e + h < n) lo = __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * (e + h), 0, kCoherent);
      if (e + h + 1 < n)
        hi = __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * (e + h + 1), 0, kCoherent);
      wd[h / 2] = lo | (hi << 16);
    }
    const uint4 v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
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

  // 5. per-round counts (ballots and scalar bit counts)
  for (int r = rw; r < R; r += RW) {
    const uint4 v = *reinterpret_cast<const uint4*>(&sm.keys[r * kRankRound + 8 * lane]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c0 = 0u, c1 = 0u, c2 = 0u, c3 = 0u;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t k = (w[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
      c0 += (uint32_t)__builtin_popcountll(__ballot(k > t1));
      c1 += (uint32_t)__builtin_popcountll(__ballot(k == t1));
      c2 += (uint32_t)__builtin_popcountll(__ballot(k > t2));
      c3 += (uint32_t)__builtin_popcountll(__ballot(k == t2));
    }
    if (lane == 0) *reinterpret_cast<uint4*>(&sm.rtot[r][0]) = make_uint4(c0, c1, c2, c3);
  }
  rank_sync<RW>(epoch, status);

  // 6. exclusive scans of the four counts over the rounds (lane l holds
  // round l), the needed rounds, then placement slot by slot
  static_assert(kRankMaxRounds <= 64, "one round per lane");
  uint32_t ex[4], own[4];
  {
    const uint4 u = lane < R ? *reinterpret_cast<const uint4*>(&sm.rtot[lane][0])
                             : make_uint4(0u, 0u, 0u, 0u);
    own[0] = u.x; own[1] = u.y; own[2] = u.z; own[3] = u.w;
#pragma unroll
    for (int q = 0; q < 4; ++q) ex[q] = wave_incl_scan(own[q]) - own[q];
  }
  const uint4 nf = *reinterpret_cast<const uint4*>(&sm.need[0]);
  const uint4 na = *reinterpret_cast<const uint4*>(&sm.need[4]);
  const uint32_t nf0 = uniform(nf.x), nf1 = uniform(nf.y), nf2 = uniform(nf.z), nf3 = uniform(nf.w);
  const uint32_t na0 = uniform(na.x), na1 = uniform(na.y), na2 = uniform(na.z), na3 = uniform(na.w);
  int32_t* out_f = uniform_ptr(reinterpret_cast<int32_t*>(sm.rank_out[0]));
  int32_t* out_a = uniform_ptr(reinterpret_cast<int32_t*>(sm.rank_out[1]));
  for (int r = rw; r < R; r += RW) {
    uint32_t G1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[0], r));
    uint32_t E1 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[1], r));
    uint32_t G2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[2], r));
    uint32_t E2 = uniform((uint32_t)__builtin_amdgcn_readlane((int)ex[3], r));
    const uint32_t G1e = G1 + (uint32_t)__builtin_amdgcn_readlane((int)own[0], r);
    const uint32_t E1e = E1 + (uint32_t)__builtin_amdgcn_readlane((int)own[1], r);
    const uint32_t G2e = G2 + (uint32_t)__builtin_amdgcn_readlane((int)own[2], r);
    const uint32_t E2e = E2 + (uint32_t)__builtin_amdgcn_readlane((int)own[3], r);
    // the round's full-tier and approx-tier position ranges
    const uint32_t fb = G1 + min(E1, q1), fe = G1e + min(E1e, q1);
    const uint32_t ab = G2 + min(E2, q2) - fb, ae = G2e + min(E2e, q2) - fe;
    const bool need = (fb < nf1 && fe > nf0) || (fb < nf3 && fe > nf2) ||
                      (ab < na1 && ae > na0) || (ab < na3 && ae > na2);
    if (!need) continue;  // wave-uniform
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t e = (uint32_t)(r * kRankRound + 64 * h + lane);
      const uint32_t k = (uint32_t)sm.keys[e] & 0x7FFFu;
      const uint64_t mg1 = __ballot(k > t1), me1 = __ballot(k == t1);
      const uint64_t mg2 = __ballot(k > t2), me2 = __ballot(k == t2);
      const uint32_t e1 = E1 + lanes_below(me1), e2 = E2 + lanes_below(me2);
      const bool in_f = k > t1 || (k == t1 && e1 < q1);
      const bool in_fa = k > t2 || (k == t2 && e2 < q2);
      const uint32_t fpos = G1 + lanes_below(mg1) + min(e1, q1);
      const uint32_t apos = G2 + lanes_below(mg2) + min(e2, q2) - fpos;
      if (in_f) {
        list[fpos] = (uint16_t)e;
        out_f[fpos] = (int32_t)e;
      } else if (in_fa) {
        list[K1 + apos] = (uint16_t)e;
        out_a[apos] = (int32_t)e;
      }
      G1 += (uint32_t)__builtin_popcountll(mg1);
      E1 += (uint32_t)__builtin_popcountll(me1);
      G2 += (uint32_t)__builtin_popcountll(mg2);
      E2 += (uint32_t)__builtin_popcountll(me2);
    }
  }
  static_assert(256 * kHistCopies == 4 * kLayerRankThreads, "one 16-byte clear per thread");
  if (rt < kLayerRankThreads) {
    reinterpret_cast<uint4*>(sm.hist)[rt] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(sm.sub)[rt] = make_uint4(0u, 0u, 0u, 0u);
  }
  rank_sync<RW>(epoch, status);
  return epoch;
}

// The positions of group g that workgroup w reads (its segments' ranges,
// two intervals per tier: a workgroup meets at most two partial tiles of a
// group, and a third tile makes the whole list needed), and the caller's
// list pointers, into LDS for the ranking.
__device__ __forceinline__ void set_need(const LayerArgs& A, int g, uint32_t w) {
  const LayerGroupArgs& gr = A.g[g];
  uint32_t f[4] = {0u, 0u, 0u, 0u}, a[4] = {0u, 0u, 0u, 0u};
  int cnt = 0;
  layer_group_segs(A, g, w, [&](const LayerSeg& s) {
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
  g_sm.rank_out[0] = reinterpret_cast<uint64_t>(gr.out_full);
  g_sm.rank_out[1] = reinterpret_cast<uint64_t>(gr.out_approx);
}

// The first group in processing order that workgroup w ranks, or -1.
__device__ __forceinline__ int first_ranked(const LayerArgs& A, uint32_t w) {
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    if (layer_meets(A, g, w) && A.g[g].k_full + A.g[g].k_approx > 0 &&
        !(g == SPAX_GROUP_DOWN && A.down_waits))
      return g;
  }
  return -1;
}

// Ranking waves: rank each further group the workgroup meets, in processing
// order (the first was ranked by the whole workgroup).
__device__ __forceinline__ void rank_role(const LayerArgs& A, int first, uint32_t epoch) {
  __builtin_amdgcn_s_setprio(3);
  uint32_t* status = A.sync + 2;
  const uint32_t w = blockIdx.x;
  const int rt = (int)threadIdx.x - (kLayerStreamWaves + 1) * 64;
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    if (g == first || !layer_meets(A, g, w)) continue;
    const LayerGroupArgs& gr = A.g[g];
    const uint32_t K1 = (uint32_t)gr.k_full, K2 = (uint32_t)(gr.k_full + gr.k_approx);
    if (K2 == 0u) continue;  // no lists: the group's segments are empty
    if (g == SPAX_GROUP_DOWN && A.down_waits) {
      // every gate/up tile has written its a (bounded wait)
      const uint32_t need = (uint32_t)A.g[SPAX_GROUP_GATE_UP].tiles;
      for (uint32_t k = 0;
           __hip_atomic_load(&A.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need;
           ++k) {
        if (k >= kSpinGlobal) {
          if ((threadIdx.x & 63) == 0) set_status(status, kStatusGlobalWait);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (rt == 0) set_need(A, g, w);
    epoch = rank_group<kLayerRankWaves>(gr.x, gr.n, K1, K2, gr.list_off, epoch, status);
    if (rt == 0)
      __hip_atomic_store(&g_sm.ready[g], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Streaming waves: per segment, this wave's share of each tier; then the
// wave's partial of the tile into LDS for the reduction wave.
template <int FF, int AF>
__device__ __forceinline__ void stream_role(const LayerArgs& A, int sw) {
  LayerShared& sm = g_sm;
  uint32_t* status = A.sync + 2;
  const int lane = (int)threadIdx.x & 63;
  const uint32_t w = blockIdx.x;
  uint32_t k = 0u;
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    layer_group_segs(A, g, w, [&](const LayerSeg& s) {
      const LayerGroupArgs& gr = A.g[g];
      const int row0 = s.t * kTileRows;
      // lanes past the last row of a ragged tile read lane 0's rows; their
      // sums are never stored
      const int ld_lane = row0 + 8 * lane < gr.rows ? lane : 0;
      float acc[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
      float corr = 0.0f;
      const int nf = s.f1 - s.f0, na = s.a1 - s.a0;
      const int flo = s.f0 + nf * sw / kNS, fhi = s.f0 + nf * (sw + 1) / kNS;
      const int alo = s.a0 + na * sw / kNS, ahi = s.a0 + na * (sw + 1) / kNS;
      if (fhi > flo || ahi > alo) {
        wait_lds_ge(&sm.ready[g], 1u, status);
        const int32_t* pl = reinterpret_cast<const int32_t*>(sm.lists + gr.list_off);
        TierStream<FF, kListPacked> sf(sm.wm[0][sw], gr.full_base, gr.full_stride, gr.full_bytes,
                                       gr.full_scales, gr.full_sstride, nullptr, gr.x, pl,
                                       nullptr, flo, fhi, row0, gr.rows, lane, ld_lane);
        sf.begin();
        if constexpr (AF != kNone) {
          const int32_t* pa =
              reinterpret_cast<const int32_t*>(sm.lists + gr.list_off + gr.k_full);
          TierStream<AF, kListPacked> sa(sm.wm[1][sw], gr.approx_base, gr.approx_stride,
                                         gr.approx_bytes, gr.approx_scales, gr.approx_sstride,
                                         nullptr, gr.x, pa, nullptr, alo, ahi, row0, gr.rows,
                                         lane, ld_lane);
          sa.begin();
          sf.run(acc, corr);
          sa.run(acc, corr);
        } else {
          sf.run(acc, corr);
        }
        if constexpr (FF == kInt4 || AF != kNone) {
#pragma unroll
          for (int r = 0; r < 8; ++r) acc[r] -= corr;
        }
      }
      // hand the partial to the reduction wave once it has read the
      // previous segment's slots
      wait_lds_ge(&sm.seg_free, k, status);
      float4* dst = reinterpret_cast<float4*>(&sm.slot[sw][8 * lane]);
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      if (lane == 0)
        __hip_atomic_fetch_add(&sm.seg_arrive, 1u, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
      ++k;
    });
  }
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

// Reduction wave: per segment, the workgroup's partial of the tile, then the
// cross-workgroup sum by the tile's last contributor.
__device__ __forceinline__ void reduce_role(const LayerArgs& A) {
  LayerShared& sm = g_sm;
  __builtin_amdgcn_s_setprio(3);
  uint32_t* status = A.sync + 2;
  const int lane = (int)threadIdx.x & 63;
  const uint32_t w = blockIdx.x;
  uint32_t k = 0u;
  for (int oi = 0; oi < A.n_order; ++oi) {
    const int g = A.order[oi];
    layer_group_segs(A, g, w, [&](const LayerSeg& s0) {
      LayerSeg s = s0;
      wait_lds_ge(&sm.seg_arrive, (uint32_t)kNS * (k + 1u), status);
      float p[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] = 0.0f;
#pragma unroll
      for (int q = 0; q < kNS; ++q) {
        const float4* src = reinterpret_cast<const float4*>(&sm.slot[q][8 * lane]);
        const float4 u0 = src[0], u1 = src[1];
        p[0] += u0.x; p[1] += u0.y; p[2] += u0.z; p[3] += u0.w;
        p[4] += u1.x; p[5] += u1.y; p[6] += u1.z; p[7] += u1.w;
      }
      ++k;
      if (lane == 0)
        __hip_atomic_store(&sm.seg_free, k, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      layer_contributors(A, s);
      if (s.w_lo == s.w_hi) {  // the only contributor
        finish_tile(A, s, p, lane);
        return;
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
      if (old != (uint32_t)(s.w_hi - s.w_lo)) return;
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
    });
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
    sm.seg_arrive = 0u;
    sm.seg_free = 0u;
  }
  // the first group the workgroup ranks: every wave ranks it (the streaming
  // waves have nothing to read before it)
  const uint32_t w = blockIdx.x;
  const int first = first_ranked(A, w);
  if (first >= 0 && t == 0) set_need(A, first, w);
  __syncthreads();
  uint32_t epoch = 0u;
  if (first >= 0) {
    const LayerGroupArgs& gr = A.g[first];
    rank_group<kWaves>(gr.x, gr.n, (uint32_t)gr.k_full, (uint32_t)(gr.k_full + gr.k_approx),
                       gr.list_off, 0u, A.sync + 2);
    if (t == 0) sm.ready[first] = 1u;
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if (wave < kLayerStreamWaves)
    stream_role<FF, AF>(A, wave);
  else if (wave == kLayerReduceWave)
    reduce_role(A);
  else
    rank_role(A, first, epoch);
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
  if (full_fmt == kFp16) {
    if (approx_fmt == kNone) return launch_pair<kFp16, kNone>(a, s);
    if (approx_fmt == kInt4) return launch_pair<kFp16, kInt4>(a, s);
    if (approx_fmt == kInt2) return launch_pair<kFp16, kInt2>(a, s);
    if (approx_fmt == kSign2) return launch_pair<kFp16, kSign2>(a, s);
  } else if (full_fmt == kInt4) {
    if (approx_fmt == kNone) return launch_pair<kInt4, kNone>(a, s);
    if (approx_fmt == kInt4) return launch_pair<kInt4, kInt4>(a, s);
    if (approx_fmt == kInt2) return launch_pair<kInt4, kInt2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spax
