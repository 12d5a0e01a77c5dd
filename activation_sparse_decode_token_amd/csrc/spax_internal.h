// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace spax {

// Rows of one workgroup tile of the tiered product: 64 lanes x 8 rows.
constexpr int kTileRows = 512;
// Waves per workgroup of the tiered product.
constexpr int kWaves = 8;
constexpr int kGemvThreads = kWaves * 64;
// Upper bound on column splits of one product (size of the fp32 partials).
constexpr int kMaxSplits = 64;
// Rows per quantisation group.
constexpr int kGroup = 128;
// List positions one workgroup of the fused rank + product keeps in LDS.
constexpr int kListCap = 2048;
// Largest input length the fused rank + product handles (64 per thread).
constexpr int kRankMaxN = kGemvThreads * 64;

enum Fmt : int32_t { kNone = 0, kFp16 = 1, kInt4 = 2, kInt2 = 3 };
enum Epi : int32_t { kEpiPlain = 0, kEpiGlu = 1 };
// Where the tiered product takes its tier lists from.
enum ListMode : int32_t {
  kListGlobal = 0,  // index lists in device memory
  kListStaged = 1,  // selected columns staged in list order
  kListRank = 2,    // every workgroup ranks x itself (fused selection)
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
  // Per column-tile byte weights used to balance the splits.
  int64_t w_full, w_approx;
  // Full tier: fp16 columns or int4 codes; column c at full_base + c * full_stride.
  const uint8_t* full_base;
  int64_t full_stride;
  const uint16_t* full_scales;   // int4 full only; column c at + c * full_sstride
  int64_t full_sstride;          // elements
  // Approx tier codes and scales.
  const uint8_t* approx_base;
  int64_t approx_stride;
  const uint16_t* approx_scales;
  int64_t approx_sstride;
  const uint16_t* x;
  const int32_t* full_idx;
  const int32_t* approx_idx;
  int32_t* out_full_idx;         // kListRank: lists written by tile-0 groups
  int32_t* out_approx_idx;
  float* partials;               // [n_splits][rows]
  uint32_t* counters;            // [n_tiles]
  uint16_t* y;                   // plain: fp16[rows]
  uint16_t* glu_a;               // glu: fp16[rows/2]
  uint16_t* glu_g;               // optional
  uint16_t* glu_u;               // optional
};

// Selected-column copy from host-resident storage into device staging.
struct CopyArgs {
  int32_t k_full, k_approx;
  int64_t e_lo, e_hi;            // virtual-list elements [e_lo, e_hi) to copy
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

hipError_t launch_gemv(const GemvArgs& a, int32_t full_fmt, int32_t approx_fmt,
                       int32_t mode, int32_t epi, hipStream_t s);

hipError_t launch_copy(const CopyArgs& a, hipStream_t s);

hipError_t launch_pack(const uint16_t* w, int32_t rows, int32_t cols, int32_t fmt,
                       uint8_t* codes, uint16_t* scales, hipStream_t s);

hipError_t launch_clear(void* ws, size_t bytes, hipStream_t s);

// First element of split s when the virtual list [full..., approx...] is cut
// into n_splits pieces of (nearly) equal bytes.
__host__ __device__ inline int64_t split_start(int64_t s, int64_t n_splits, int64_t kf,
                                               int64_t ka, int64_t wf, int64_t wa) {
  const int64_t ftot = kf * wf;
  const int64_t tot = ftot + ka * wa;
  if (s <= 0) return 0;
  if (s >= n_splits) return kf + ka;
  const int64_t B = (tot * s) / n_splits;
  if (B <= ftot) return wf > 0 ? (B + wf - 1) / wf : 0;
  return kf + (wa > 0 ? (B - ftot + wa - 1) / wa : ka);
}

}  // namespace spax
