// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace spax {

// Rows of one workgroup tile of the tiered product: 64 lanes x 8 rows.
constexpr int kTileRows = 512;
// Waves per workgroup of the tiered product.
#ifndef SPAX_WAVES
#define SPAX_WAVES 16
#endif
constexpr int kWaves = SPAX_WAVES;
constexpr int kGemvThreads = kWaves * 64;
// Upper bound on column splits of one product (size of the fp32 partials).
constexpr int kMaxSplits = 64;
// Arrival counters per row tile: one total and one per group of 8 splits.
constexpr int kCountersPerTile = 1 + kMaxSplits / 8;
// Largest matrix height and its row tiles. The counters of every matrix
// occupy one fixed region at the start of the workspace, so matrices of
// different heights can share a workspace without their partial sums
// landing on each other's counters.
constexpr int kMaxRows = 1 << 20;
constexpr int kMaxTiles = kMaxRows / kTileRows;
constexpr size_t kCounterRegionBytes = sizeof(uint32_t) * kCountersPerTile * kMaxTiles;
// Rows per quantisation group.
constexpr int kGroup = 128;
// List positions one workgroup of the fused rank + product keeps in LDS.
constexpr int kListCap = 2048;
// The same with the trellis tier, whose 128 KB codebook shares the LDS.
constexpr int kListCapTrellis = 1024;
// Largest input length the fused rank + product handles (8 ranking waves,
// up to 64 entries per ranking thread); longer inputs are ranked by the
// sliced selection kernels first. Measured at n = 28672 (70B down): the
// fused form is faster now that its histograms run on the ranking waves
// only; the sliced form's three launches cost about 14 us of latency.
constexpr int kRankMaxN = kGemvThreads * 32;
// Sliced selection: entries per slice (one workgroup, 4 per thread) and the
// most slices (inputs up to 65536 entries).
constexpr int kSliceEntries = kGemvThreads * 4;
constexpr int kMaxSlices = 65536 / kSliceEntries;

enum Fmt : int32_t { kNone = 0, kFp16 = 1, kInt4 = 2, kInt2 = 3, kSign2 = 4, kTrellis = 5 };
enum Epi : int32_t { kEpiPlain = 0, kEpiGlu = 1 };
// Where the tiered product takes its tier lists from.
enum ListMode : int32_t {
  kListGlobal = 0,  // index lists in device memory
  kListStaged = 1,  // selected columns staged in list order
  kListRank = 2,    // every workgroup ranks x itself (fused selection)
  kListSliced = 3,  // thresholds and slice counts from the sliced selection;
                    // every workgroup places its piece from its slices
  kListPacked = 4,  // the layer kernel's whole ranked lists in LDS, 16-bit
                    // column indices; activations read from the input
};

// Arguments of one launch of the tiered product.
struct GemvArgs {
  int32_t rows;                  // stored rows R
  int32_t n_tiles;               // ceil(R / kTileRows)
  int32_t n_splits;              // column splits of the whole product
  int32_t split_lo;              // first split handled by this launch
  int32_t splits_here;           // splits handled by this launch
  int32_t k_full, k_approx;
  int32_t n;                     // input length (cols)
  // Full tier: fp16 columns or int4 codes; column c at full_base + c * full_stride.
  const uint8_t* full_base;
  int64_t full_stride;
  uint32_t full_bytes;           // bytes of the full tier (< 2^31)
  uint32_t approx_bytes;         // bytes of the approx codes (< 2^31)
  const uint16_t* full_scales;   // int4 full only; column c at + c * full_sstride
  int64_t full_sstride;          // elements
  // Approx tier codes and scales.
  const uint8_t* approx_base;
  int64_t approx_stride;
  const uint16_t* approx_scales;
  int64_t approx_sstride;
  // Matrices in a stored column of a sign / trellis approx tier: 0 one,
  // S > 0 stacked segments of S rows (S % 512 == 0), -1 GLU gate and up
  // (128-row blocks by parity); approx_nseg their number.
  int32_t approx_seg, approx_nseg;
  const uint16_t* x;
  const int32_t* full_idx;
  const int32_t* approx_idx;
  int32_t* out_full_idx;         // kListRank: lists written by tile-0 groups
  int32_t* out_approx_idx;
  float* partials;               // [n_splits][rows]
  uint32_t* counters;            // [n_tiles][kCountersPerTile]
  uint16_t* y;                   // plain: fp16[rows]
  uint16_t* glu_a;               // glu: fp16[rows/2]
  uint16_t* glu_g;               // optional
  uint16_t* glu_u;               // optional
  const struct SelectScratch* sel;  // kListSliced: thresholds and slice counts
  int32_t slices;                // kListSliced: slices of x
  const uint16_t* codebook;      // trellis approx tier: fp16[65536]
};

// Workspace region of the sliced selection: per-slice histograms and counts,
// and the selection results (b1, entries above b1, b2, entries above b2,
// t1, q1, t2, q2). Every field is written before it is read in each call.
struct SelectScratch {
  uint32_t hist[kMaxSlices][256];
  uint32_t sub[kMaxSlices][2][128];
  uint32_t cnt[kMaxSlices][4];
  int32_t sel[8];
};

// Selected-column copy from host-resident storage into device staging.
struct CopyArgs {
  int32_t k_full, k_approx;
  int32_t f_lo, f_hi;            // full-tier list positions [f_lo, f_hi) to copy
  int32_t a_lo, a_hi;            // approx-tier list positions [a_lo, a_hi) to copy
  const int32_t* full_idx;
  const int32_t* approx_idx;
  // sources (host pinned, device addressable)
  const uint8_t* full_src;   int64_t full_bytes;     // bytes per full column
  const uint16_t* fscale_src; int32_t fscale_n;      // scales per full column (0 if none)
  const uint8_t* approx_src; int64_t approx_bytes;   // bytes per approx column
  const uint16_t* ascale_src; int32_t ascale_n;      // scales per approx column
  // destinations (device staging, indexed by list position)
  uint8_t* full_dst; uint16_t* fscale_dst;
  uint8_t* approx_dst; uint16_t* ascale_dst;
};

hipError_t launch_plan(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                       int32_t* full_idx, int32_t* approx_idx, hipStream_t s);

// Sliced selection of x (n <= 65536): thresholds and per-slice counts into
// ws; with lists (full_idx non-null) also the ascending full / approx lists.
hipError_t launch_select(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                         int32_t* full_idx, int32_t* approx_idx, SelectScratch* ws,
                         hipStream_t s);

hipError_t launch_gemv(const GemvArgs& a, int32_t full_fmt, int32_t approx_fmt,
                       int32_t mode, int32_t epi, hipStream_t s);

hipError_t launch_copy(const CopyArgs& a, hipStream_t s);

hipError_t launch_pack(const uint16_t* w, int32_t rows, int32_t cols, int32_t fmt,
                       uint8_t* codes, uint16_t* scales, hipStream_t s);

hipError_t launch_pack_sign2(const uint16_t* w, int32_t rows, int32_t cols, uint8_t* codes,
                             uint16_t* scales, hipStream_t s);

// Trellis encoder: backpointer workspace per column in flight, and the
// launches (columns in batches that fit the workspace).
size_t trellis_ws_per_column(int32_t rows);
hipError_t launch_pack_trellis(const uint16_t* w, int32_t rows, int32_t cols,
                               const uint16_t* codebook, uint8_t* codes, uint16_t* scales,
                               void* ws, size_t ws_bytes, hipStream_t s);

hipError_t launch_clear(void* ws, size_t bytes, hipStream_t s);
hipError_t launch_sq_error(const uint16_t* y, const uint16_t* r, int64_t n, double* acc,
                           int32_t accumulate, hipStream_t s);
// Bytes at the start of a workspace that must start at zero (arrival
// counters, the layer kernel's sync words, the sliced selection's counts).
size_t workspace_head_bytes();
// Sets the text spax_last_error returns on this thread.
void set_last_error(const char* msg);

// List positions of split s of n_splits: every split takes the same share
// of each tier, [k * s / n_splits, k * (s + 1) / n_splits), so every
// workgroup gets the same mix of full columns (bytes) and code columns
// (bytes plus dequantisation arithmetic). 32-bit arithmetic: k * n_splits
// stays below 2^32 (k <= columns, which are below 2^26 since a tier holds
// under 2^31 bytes of at least 32-byte columns, and n_splits <= 64).
__host__ __device__ inline int32_t split_pos(uint32_t s, uint32_t n_splits, uint32_t k) {
  return (int32_t)(k * s / n_splits);
}

}  // namespace spax
