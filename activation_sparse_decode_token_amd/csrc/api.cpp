// C ABI of the three-tier activation-sparse decode library: argument
// validation, launch planning, workspace layout and the layer sequence.
// All arithmetic of the method runs in the kernels (plan.hip, select.hip,
// gemv.hip, layer.hip, aux.hip); this file only checks arguments, plans
// launches and enqueues work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <string>

#include "layer_plan.h"
#include "spax.h"
#include "spax_internal.h"

namespace {

using namespace spax;

thread_local std::string g_last_error = "no error";

int hip_fail(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return SPAX_EHIP;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Bytes of one stored column (codes only for code formats).
int64_t col_bytes(int32_t fmt, int64_t rows) {
  switch (fmt) {
    case kFp16: return 2 * rows;
    case kInt4: return rows / 2;
    case kInt2: return rows / 4;
    case kSign2: return rows / 4;
    case kTrellis: return rows / 4;
    default: return 0;
  }
}
// fp16 scales per stored column (0 for fp16 values; 2 for the sign code).
int64_t col_scales(int32_t fmt, int64_t rows) {
  if (fmt == kSign2) return 2;
  if (fmt == kTrellis) return 1;
  return (fmt == kInt4 || fmt == kInt2) ? rows / kGroup : 0;
}
// Matrices in one stored column of a sign / trellis approx tier, each coded
// as its own column: gate and up in the GLU layout, else rows /
// approx_seg_rows stacked segments (one when 0).
int32_t approx_nseg(const spax_matrix* W) {
  if (W->layout == SPAX_LAYOUT_GLU_INTERLEAVED) return 2;
  return W->approx_seg_rows > 0 ? W->rows / W->approx_seg_rows : 1;
}
// The kernels' segment mode: 0 one matrix, S stacked segments of S rows,
// -1 GLU gate/up blocks.
int32_t approx_seg_mode(const spax_matrix* W) {
  if (W->approx_fmt != kSign2 && W->approx_fmt != kTrellis) return 0;
  if (W->layout == SPAX_LAYOUT_GLU_INTERLEAVED) return -1;
  return W->approx_seg_rows;
}
// fp16 scales per stored column of the approx tier.
int64_t approx_col_scales(const spax_matrix* W) {
  if (W->approx_fmt == kSign2) return 2 * approx_nseg(W);
  if (W->approx_fmt == kTrellis) return approx_nseg(W);
  return col_scales(W->approx_fmt, W->rows);
}
// Bytes one 512-row tile of a column costs, used to balance the splits.
int64_t tile_bytes(int32_t fmt) {
  switch (fmt) {
    case kFp16: return 2 * kTileRows;
    case kInt4: return kTileRows / 2 + 2 * (kTileRows / kGroup);
    case kInt2: return kTileRows / 4 + 2 * (kTileRows / kGroup);
    case kSign2: return kTileRows / 4 + 4;
    case kTrellis: return kTileRows / 4 + 2;
    default: return 0;
  }
}

int validate_matrix(const spax_matrix* W) {
  if (!W) return SPAX_ENULL;
  if (W->rows <= 0 || W->cols <= 0 || W->rows % kGroup || W->rows > kMaxRows)
    return SPAX_EINVAL;
  if (W->full_fmt != kFp16 && W->full_fmt != kInt4) return SPAX_EFORMAT;
  if (W->approx_fmt != kNone && W->approx_fmt != kInt4 && W->approx_fmt != kInt2 &&
      W->approx_fmt != kSign2 && W->approx_fmt != kTrellis)
    return SPAX_EFORMAT;
  if ((W->approx_fmt == kSign2 || W->approx_fmt == kTrellis) && W->full_fmt != kFp16)
    return SPAX_EFORMAT;
  if (W->approx_fmt == kTrellis) {
    if (!W->approx_codebook) return SPAX_ENULL;
    if (!aligned16(W->approx_codebook)) return SPAX_EALIGN;
  }
  if (W->residency != SPAX_RES_DEVICE && W->residency != SPAX_RES_HOST_PINNED)
    return SPAX_EINVAL;
  if (W->layout != SPAX_LAYOUT_PLAIN && W->layout != SPAX_LAYOUT_GLU_INTERLEAVED)
    return SPAX_EINVAL;
  if (W->layout == SPAX_LAYOUT_GLU_INTERLEAVED && W->rows % (2 * kGroup)) return SPAX_EINVAL;
  // stacked matrices: whole 512-row tiles each, so a tile never holds two
  if (W->approx_seg_rows < 0) return SPAX_EINVAL;
  if (W->approx_seg_rows > 0 &&
      (W->layout != SPAX_LAYOUT_PLAIN || W->approx_seg_rows % kTileRows ||
       W->rows % W->approx_seg_rows))
    return SPAX_EINVAL;
  // the product addresses each tier with 32-bit offsets
  if (col_bytes(W->full_fmt, W->rows) * W->cols >= (int64_t(1) << 31) ||
      col_bytes(W->approx_fmt, W->rows) * W->cols >= (int64_t(1) << 31))
    return SPAX_EINVAL;
  if (!W->full_data) return SPAX_ENULL;
  if (W->full_fmt == kInt4 && !W->full_scales) return SPAX_ENULL;
  if (W->approx_fmt != kNone && (!W->approx_codes || !W->approx_scales)) return SPAX_ENULL;
  if (!aligned16(W->full_data) || !aligned16(W->full_scales) || !aligned16(W->approx_codes) ||
      !aligned16(W->approx_scales))
    return SPAX_EALIGN;
  return SPAX_OK;
}

struct ProductPlan {
  int32_t tiles = 1;
  int32_t splits = 1;
};

#ifndef SPAX_TARGET_BLOCKS
#define SPAX_TARGET_BLOCKS 256
#endif
#ifndef SPAX_MIN_SPLIT_BYTES
#define SPAX_MIN_SPLIT_BYTES 32768
#endif

// Number of column splits: at most one 16-wave workgroup per compute unit
// (tiles x splits <= SPAX_TARGET_BLOCKS, so the grid runs in one pass), at
// least SPAX_MIN_SPLIT_BYTES of weights per workgroup.
ProductPlan plan_product(const spax_matrix* W, int32_t kf, int32_t ka) {
  constexpr int64_t kTargetBlocks = SPAX_TARGET_BLOCKS;
  constexpr int64_t kMinSplitBytes = SPAX_MIN_SPLIT_BYTES;
  ProductPlan p;
  p.tiles = (W->rows + kTileRows - 1) / kTileRows;
  const int64_t total = kf * tile_bytes(W->full_fmt) + ka * tile_bytes(W->approx_fmt);
  if (total == 0) return p;
  int64_t s = std::max<int64_t>(1, kTargetBlocks / p.tiles);
  s = std::min<int64_t>(s, std::max<int64_t>(1, total / kMinSplitBytes));
  s = std::min<int64_t>(s, kMaxSplits);
  s = std::min<int64_t>(s, (int64_t)kf + ka);
  p.splits = (int32_t)std::max<int64_t>(1, s);
  return p;
}

// Largest number of list positions one split holds.
int64_t max_piece(const ProductPlan& p, int32_t kf, int32_t ka) {
  int64_t m = 0;
  for (int s = 0; s < p.splits; ++s)
    m = std::max<int64_t>(m, split_pos(s + 1, p.splits, kf) - split_pos(s, p.splits, kf) +
                                 split_pos(s + 1, p.splits, ka) - split_pos(s, p.splits, ka));
  return m;
}

// Plan of a product whose workgroups keep their list piece in LDS (fused
// rank, or placement from the sliced selection): more splits while a piece
// would not fit. Returns false when no split count fits.
bool plan_piece(const spax_matrix* W, int32_t kf, int32_t ka, ProductPlan* out) {
  if (W->residency != SPAX_RES_DEVICE) return false;
  // the trellis tier's codebook leaves room for a smaller piece
  const int64_t cap = W->approx_fmt == kTrellis ? kListCapTrellis : kListCap;
  ProductPlan p = plan_product(W, kf, ka);
  while (max_piece(p, kf, ka) > cap) {
    if (p.splits >= kMaxSplits || p.splits >= (int64_t)kf + ka) return false;
    p.splits = (int32_t)std::min<int64_t>({(int64_t)p.splits * 2, kMaxSplits, (int64_t)kf + ka});
  }
  *out = p;
  return true;
}

// Workspace layout (every region at a fixed place, so one workspace sized
// for the largest matrix serves any mix of calls):
//   [arrival counters][layer-kernel sync words][sliced-selection scratch]
//   [fp32 partial sums][host-resident staging]
size_t counters_bytes() { return align256(kCounterRegionBytes); }
constexpr size_t kSyncBytes = 256;
constexpr size_t kSelectBytes = (sizeof(SelectScratch) + 255) & ~size_t(255);
uint32_t* sync_words(void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + counters_bytes());
}
SelectScratch* select_scratch(void* ws) {
  return reinterpret_cast<SelectScratch*>(static_cast<uint8_t*>(ws) + counters_bytes() +
                                          kSyncBytes);
}
size_t partials_offset() { return counters_bytes() + kSyncBytes + kSelectBytes; }

}  // namespace

namespace spax {
size_t workspace_head_bytes() { return partials_offset(); }
void set_last_error(const char* msg) { g_last_error = msg; }
}  // namespace spax

namespace {
size_t partials_bytes(const spax_matrix* W) {
  return align256(sizeof(float) * (size_t)kMaxSplits * W->rows);
}
size_t staging_bytes(const spax_matrix* W) {
  if (W->residency != SPAX_RES_HOST_PINNED) return 0;
  const int64_t per_full = col_bytes(W->full_fmt, W->rows) + 2 * col_scales(W->full_fmt, W->rows);
  const int64_t per_apx =
      col_bytes(W->approx_fmt, W->rows) + 2 * approx_col_scales(W);
  return align256((size_t)W->cols * std::max(per_full, per_apx)) + 4 * 256;
}
size_t gemv_ws(const spax_matrix* W) {
  return partials_offset() + partials_bytes(W) + staging_bytes(W);
}

// ---- the layer kernel (one launch per layer step) --------------------------

// Smallest share of a group's selected bytes worth one workgroup.
constexpr uint64_t kLayerMinWgBytes = 32768;

int32_t row_tiles(int32_t rows) { return (rows + kTileRows - 1) / kTileRows; }

// Partial-sum bytes of one group in the layer kernel (any workgroup count).
size_t layer_group_partials(const spax_matrix* W) {
  return align256(sizeof(float) * kTileRows * (size_t)(row_tiles(W->rows) + kLayerMaxWgs));
}
size_t layer_ws(const spax_layer* L) {
  size_t b = partials_offset();
  for (int g = 0; g < 4; ++g)
    if (L->group[g].cols > 0) b += layer_group_partials(&L->group[g]);
  return b;
}

// Whether the layer kernel runs L: every present group device-resident, one
// format pair (not the trellis code), inputs up to kLayerMaxN and every
// group's lists in LDS together.
bool layer_fits(const spax_layer* L, int32_t* ff, int32_t* af) {
  int present = 0;
  int64_t words = 0;
  for (int g = 0; g < 4; ++g) {
    const spax_matrix& M = L->group[g];
    if (M.cols <= 0) continue;
    if (M.residency != SPAX_RES_DEVICE || M.cols > kLayerMaxN) return false;
    if (present == 0) {
      *ff = M.full_fmt;
      *af = M.approx_fmt;
    } else if (M.full_fmt != *ff || M.approx_fmt != *af) {
      return false;
    }
    words += (int64_t)L->k_full[g] + L->k_approx[g];
    ++present;
  }
  if (present == 0 || *af == kTrellis) return false;
  // code-only layers (an int4 full tier): the per-group launches, where all
  // 16 waves of a workgroup stream the codes, measured faster (70B FFN
  // layer: 73.8 against 84.5 us per layer step)
  if (*ff == kInt4) return false;
  return words <= kLayerListCap;
}

// Bytes of the selected columns of group g over all its row tiles.
uint64_t layer_group_bytes(const spax_layer* L, int g) {
  const spax_matrix& M = L->group[g];
  return (uint64_t)row_tiles(M.rows) *
         ((uint64_t)L->k_full[g] * tile_bytes(M.full_fmt) +
          (uint64_t)L->k_approx[g] * tile_bytes(M.approx_fmt));
}

// Schedule fields of the layer kernel's arguments (no pointers) for at most
// Gmax workgroups: gate/up and down on all of them, q/k/v and o on two
// disjoint ranges in proportion to their bytes; no group on more workgroups
// than it has units or kLayerMinWgBytes shares of its bytes. A->G is the
// number of workgroups used.
void layer_schedule(const spax_layer* L, int32_t Gmax, LayerArgs* A) {
  *A = LayerArgs{};
  const bool has_gu = L->group[SPAX_GROUP_GATE_UP].cols > 0;
  int32_t list_off = 0;
  for (int oi = 0; oi < 4; ++oi) {
    const int g = layer_order(oi);
    const spax_matrix& M = L->group[g];
    if (M.cols <= 0) continue;
    LayerGroupArgs& gr = A->g[g];
    gr.present = 1;
    gr.rows = M.rows;
    gr.n = M.cols;
    gr.k_full = L->k_full[g];
    gr.k_approx = L->k_approx[g];
    gr.tiles = row_tiles(M.rows);
    gr.list_off = list_off;
    list_off += gr.k_full + gr.k_approx;
    A->order[A->n_order++] = g;
  }
  A->down_waits = has_gu && L->group[SPAX_GROUP_DOWN].cols > 0;
  // the workgroup ranges
  int64_t lo[4] = {0, 0, 0, 0}, span[4] = {Gmax, Gmax, Gmax, Gmax};
  const uint64_t bq = A->g[SPAX_GROUP_QKV].present ? layer_group_bytes(L, SPAX_GROUP_QKV) : 0;
  const uint64_t bo = A->g[SPAX_GROUP_O].present ? layer_group_bytes(L, SPAX_GROUP_O) : 0;
  if (bq > 0 && bo > 0 && Gmax >= 2) {
    const int64_t sq = std::min<int64_t>(
        Gmax - 1, std::max<int64_t>(1, (int64_t)((Gmax * (double)bq) / (double)(bq + bo) + 0.5)));
    span[SPAX_GROUP_QKV] = sq;
    span[SPAX_GROUP_O] = Gmax - sq;
  }
  int64_t G = 1;
  for (int oi = 0; oi < A->n_order; ++oi) {
    const int g = A->order[oi];
    LayerGroupArgs& gr = A->g[g];
    const uint64_t K = (uint64_t)gr.k_full + gr.k_approx;
    gr.units = (uint32_t)((uint64_t)gr.tiles * K);
    if (gr.units == 0) {  // tiles dealt round-robin over every workgroup
      gr.wg_lo = 0;
      gr.n_wg = 0;
      G = std::max<int64_t>(G, std::min<int64_t>(Gmax, gr.tiles));
      continue;
    }
    const int64_t want = std::max<int64_t>(1, (int64_t)(layer_group_bytes(L, g) / kLayerMinWgBytes));
    const int64_t n = std::min<int64_t>({span[g], want, (int64_t)gr.units});
    if (g == SPAX_GROUP_O && span[SPAX_GROUP_QKV] < Gmax)
      lo[g] = A->g[SPAX_GROUP_QKV].wg_lo + A->g[SPAX_GROUP_QKV].n_wg;
    gr.wg_lo = (int32_t)lo[g];
    gr.n_wg = (int32_t)n;
    gr.unit_q = gr.units / (uint32_t)n;
    gr.unit_r = gr.units % (uint32_t)n;
    gr.k_magic = div_magic((uint32_t)K);
    gr.nwg_magic = div_magic((uint32_t)n);
    G = std::max<int64_t>(G, lo[g] + n);
  }
  A->G = (int32_t)G;
}

// Workgroups the layer kernel may use on a device: one per compute unit.
int32_t layer_workgroups(int32_t cus) {
  return std::max<int32_t>(1, std::min<int32_t>(cus, kLayerMaxWgs));
}

// Compute units of the current device (queried once per device).
std::atomic<int32_t> g_cus[64];
int device_cus(int32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < 64) {
    const int32_t v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return SPAX_OK;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  if (v <= 0) return hip_fail(hipErrorInvalidDevice);
  if (dev >= 0 && dev < 64) g_cus[dev].store(v, std::memory_order_relaxed);
  *out = v;
  return SPAX_OK;
}

// Whether every workgroup of schedule A stays within its segment table in
// both phases (the second: down, when gate/up runs in the same launch).
bool layer_segs_fit(const LayerArgs& A) {
  auto late = [&](int g) { return g == SPAX_GROUP_DOWN && A.down_waits; };
  return layer_phase_segs_bound(A, [&](int g) { return !late(g); }) <= (uint32_t)kLayerSegTab &&
         layer_phase_segs_bound(A, late) <= (uint32_t)kLayerSegTab;
}

// The layer kernel's launch for L on the current device, or *ok = false
// when a workgroup could meet more segments than its table holds.
int plan_layer_kernel(const spax_layer* L, LayerArgs* A, bool* ok) {
  int32_t cus = 0;
  const int st = device_cus(&cus);
  if (st) return st;
  const int32_t G = layer_workgroups(cus);
  layer_schedule(L, L->workgroups > 0 ? std::min(L->workgroups, G) : G, A);
  *ok = layer_segs_fit(*A);
  return SPAX_OK;
}

int run_layer_kernel(const spax_layer* L, const spax_layer_io* io, void* ws, int32_t ff,
                     int32_t af, LayerArgs& A, hipStream_t s) {
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  size_t poff = partials_offset();
  const uint16_t* inputs[4] = {io->h, io->z, io->x, io->a};
  uint16_t* outputs[4] = {io->qkv, io->o, nullptr, io->down};
  for (int g = 0; g < 4; ++g) {
    const spax_matrix& M = L->group[g];
    if (M.cols <= 0) continue;
    LayerGroupArgs& gr = A.g[g];
    const int64_t fb = col_bytes(M.full_fmt, M.rows), ab = col_bytes(M.approx_fmt, M.rows);
    gr.full_base = static_cast<const uint8_t*>(M.full_data);
    gr.full_stride = fb;
    gr.full_bytes = (uint32_t)(fb * M.cols);
    gr.full_scales = M.full_scales;
    gr.full_sstride = col_scales(M.full_fmt, M.rows);
    gr.approx_base = M.approx_codes;
    gr.approx_stride = ab;
    gr.approx_bytes = (uint32_t)(ab * M.cols);
    gr.approx_scales = M.approx_scales;
    gr.approx_sstride = approx_col_scales(&M);
    gr.approx_seg = approx_seg_mode(&M);
    gr.approx_nseg = approx_nseg(&M);
    gr.x = inputs[g];
    gr.y = outputs[g];
    gr.out_full = io->full_idx[g];
    gr.out_approx = io->approx_idx[g];
    gr.partials = reinterpret_cast<float*>(wsb + poff);
    poff += layer_group_partials(&M);
    gr.counters = reinterpret_cast<uint32_t*>(wsb) + g;
  }
  A.glu_a = io->a;
  A.glu_g = io->g;
  A.glu_u = io->u;
  A.sync = sync_words(ws);
  const hipError_t e = launch_layer(A, ff, af, s);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

// The copy context of a host-resident call: set up, on the current device.
int check_copy(const spax_copy* cp) {
  if (!cp || !cp->stream || !cp->ready) return SPAX_ESTREAM;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  return dev == cp->device ? SPAX_OK : SPAX_ESTREAM;
}

// Enqueue one tiered product. mode kListRank ranks x inside the product and
// writes the lists to out_f / out_a; the other modes read fidx / aidx.
int run_product(const spax_matrix* W, const uint16_t* x, const int32_t* fidx, int32_t kf,
                const int32_t* aidx, int32_t ka, int32_t epi, uint16_t* y, uint16_t* ga,
                uint16_t* gg, uint16_t* gu, void* ws, hipStream_t s, const spax_copy* cp,
                const ProductPlan* piece = nullptr, int32_t piece_mode = kListRank,
                int32_t* out_f = nullptr,
                int32_t* out_a = nullptr) {
  const ProductPlan p = piece ? *piece : plan_product(W, kf, ka);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  GemvArgs a{};
  a.rows = W->rows;
  a.n_tiles = p.tiles;
  a.n_splits = p.splits;
  a.k_full = kf;
  a.k_approx = ka;
  a.n = W->cols;
  a.x = x;
  a.full_idx = fidx;
  a.approx_idx = aidx;
  a.out_full_idx = out_f;
  a.out_approx_idx = out_a;
  a.sel = select_scratch(ws);
  a.slices = (W->cols + kSliceEntries - 1) / kSliceEntries;
  a.counters = reinterpret_cast<uint32_t*>(wsb);
  a.partials = reinterpret_cast<float*>(wsb + partials_offset());
  a.y = y;
  a.glu_a = ga;
  a.glu_g = gg;
  a.glu_u = gu;
  a.codebook = W->approx_codebook;
  const int64_t fb = col_bytes(W->full_fmt, W->rows), fsn = col_scales(W->full_fmt, W->rows);
  const int64_t ab = col_bytes(W->approx_fmt, W->rows), asn = approx_col_scales(W);
  a.full_stride = fb;
  a.full_sstride = fsn;
  a.approx_stride = ab;
  a.approx_sstride = asn;
  a.approx_seg = approx_seg_mode(W);
  a.approx_nseg = approx_nseg(W);
  // bytes the product may read from each tier (the staging holds the
  // selected columns in list order)
  const bool staged = W->residency == SPAX_RES_HOST_PINNED;
  a.full_bytes = (uint32_t)(fb * (staged ? kf : W->cols));
  a.approx_bytes = (uint32_t)(ab * (staged ? ka : W->cols));

  if (W->residency == SPAX_RES_DEVICE) {
    a.full_base = static_cast<const uint8_t*>(W->full_data);
    a.full_scales = W->full_scales;
    a.approx_base = W->approx_codes;
    a.approx_scales = W->approx_scales;
    a.split_lo = 0;
    a.splits_here = p.splits;
    const hipError_t e =
        launch_gemv(a, W->full_fmt, W->approx_fmt, piece ? piece_mode : kListGlobal, epi, s);
    return e == hipSuccess ? SPAX_OK : hip_fail(e);
  }

  // Host-resident: copy the selected columns into staging in chunks on the
  // copy stream; the product consumes each chunk's splits as it lands.
  uint8_t* st = wsb + partials_offset() + partials_bytes(W);
  size_t off = 0;
  uint8_t* full_dst = st + off;
  off = align256(off + (size_t)kf * fb);
  uint16_t* fscale_dst = reinterpret_cast<uint16_t*>(st + off);
  off = align256(off + (size_t)kf * fsn * 2);
  uint8_t* approx_dst = st + off;
  off = align256(off + (size_t)ka * ab);
  uint16_t* ascale_dst = reinterpret_cast<uint16_t*>(st + off);

  a.full_base = full_dst;
  a.full_scales = fscale_dst;
  a.approx_base = approx_dst;
  a.approx_scales = ascale_dst;

  CopyArgs c{};
  c.k_full = kf;
  c.k_approx = ka;
  c.full_idx = fidx;
  c.approx_idx = aidx;
  c.full_src = static_cast<const uint8_t*>(W->full_data);
  c.full_bytes = fb;
  c.fscale_src = W->full_scales;
  c.fscale_n = (int32_t)fsn;
  c.approx_src = W->approx_codes;
  c.approx_bytes = ab;
  c.ascale_src = W->approx_scales;
  c.ascale_n = (int32_t)asn;
  c.full_dst = full_dst;
  c.fscale_dst = fscale_dst;
  c.approx_dst = approx_dst;
  c.ascale_dst = ascale_dst;

  // the lists (and the previous use of the staging) are ready on `s`
  const hipStream_t cs = cp->stream;
  hipError_t e;
  if ((e = hipEventRecord(cp->ready, s)) != hipSuccess) return hip_fail(e);
  if ((e = hipStreamWaitEvent(cs, cp->ready, 0)) != hipSuccess) return hip_fail(e);
  const int chunks = std::min(SPAX_COPY_CHUNKS, p.splits);
  for (int k = 0; k < chunks; ++k) {
    const int s_lo = (int)((int64_t)p.splits * k / chunks);
    const int s_hi = (int)((int64_t)p.splits * (k + 1) / chunks);
    c.f_lo = split_pos(s_lo, p.splits, kf);
    c.f_hi = split_pos(s_hi, p.splits, kf);
    c.a_lo = split_pos(s_lo, p.splits, ka);
    c.a_hi = split_pos(s_hi, p.splits, ka);
    if ((e = launch_copy(c, cs)) != hipSuccess) return hip_fail(e);
    if ((e = hipEventRecord(cp->chunk[k], cs)) != hipSuccess) return hip_fail(e);
    if ((e = hipStreamWaitEvent(s, cp->chunk[k], 0)) != hipSuccess) return hip_fail(e);
    a.split_lo = s_lo;
    a.splits_here = s_hi - s_lo;
    if ((e = launch_gemv(a, W->full_fmt, W->approx_fmt, kListStaged, epi, s)) != hipSuccess)
      return hip_fail(e);
  }
  return SPAX_OK;
}

int check_counts(int32_t n, int32_t kf, int32_t ka) {
  if (kf < 0 || ka < 0 || (int64_t)kf + ka > n) return SPAX_EINVAL;
  return SPAX_OK;
}

int validate_product(const spax_matrix* W, const uint16_t* x, const int32_t* fidx, int32_t kf,
                     const int32_t* aidx, int32_t ka, const void* ws, size_t ws_bytes,
                     const spax_copy* cp) {
  int st = validate_matrix(W);
  if (st) return st;
  if ((st = check_counts(W->cols, kf, ka))) return st;
  if (ka > 0 && W->approx_fmt == kNone) return SPAX_EINVAL;
  if (!x || (kf > 0 && !fidx) || (ka > 0 && !aidx) || !ws) return SPAX_ENULL;
  if (!aligned16(x) || !aligned16(fidx) || !aligned16(aidx) || !aligned16(ws)) return SPAX_EALIGN;
  if (ws_bytes < gemv_ws(W)) return SPAX_EWORKSPACE;
  if (W->residency == SPAX_RES_HOST_PINNED) return check_copy(cp);
  return SPAX_OK;
}

}  // namespace

extern "C" {

int spax_version(void) { return 200; }

const char* spax_status_string(int status) {
  switch (status) {
    case SPAX_OK: return "ok";
    case SPAX_EINVAL: return "invalid size or tier count";
    case SPAX_ENULL: return "required pointer is null";
    case SPAX_EALIGN: return "device pointer is not 16-byte aligned";
    case SPAX_EFORMAT: return "unknown or unsupported format";
    case SPAX_EWORKSPACE: return "workspace too small";
    case SPAX_ESTREAM: return "host-resident matrix needs a copy set up on this device";
    case SPAX_EHIP: return "HIP runtime error";
    case SPAX_ENOMEM: return "host memory for scratch could not be allocated";
    default: return "unknown status";
  }
}

const char* spax_last_error(void) { return g_last_error.c_str(); }

int spax_copy_init(spax_copy* copy, hipStream_t copy_stream) {
  if (!copy || !copy_stream) return SPAX_ENULL;
  *copy = spax_copy{};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  spax_copy c{};
  c.stream = copy_stream;
  c.device = dev;
  e = hipEventCreateWithFlags(&c.ready, hipEventDisableTiming);
  for (int k = 0; e == hipSuccess && k < SPAX_COPY_CHUNKS; ++k)
    e = hipEventCreateWithFlags(&c.chunk[k], hipEventDisableTiming);
  if (e != hipSuccess) {
    spax_copy_release(&c);
    return hip_fail(e);
  }
  *copy = c;
  return SPAX_OK;
}

int spax_copy_release(spax_copy* copy) {
  if (!copy) return SPAX_ENULL;
  hipError_t first = hipSuccess;
  auto drop = [&](hipEvent_t& ev) {
    if (ev) {
      const hipError_t e = hipEventDestroy(ev);
      if (first == hipSuccess) first = e;
      ev = nullptr;
    }
  };
  drop(copy->ready);
  for (auto& c : copy->chunk) drop(c);
  copy->stream = nullptr;
  return first == hipSuccess ? SPAX_OK : hip_fail(first);
}

int spax_plan_tiers(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                    int32_t* full_idx, int32_t* approx_idx, hipStream_t stream) {
  if (n < 1 || n > 65536) return SPAX_EINVAL;
  int st = check_counts(n, k_full, k_approx);
  if (st) return st;
  if (!x || (k_full > 0 && !full_idx) || (k_approx > 0 && !approx_idx)) return SPAX_ENULL;
  if (!aligned16(x) || !aligned16(full_idx) || !aligned16(approx_idx)) return SPAX_EALIGN;
  const hipError_t e = launch_plan(x, n, k_full, k_approx, full_idx, approx_idx, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

size_t spax_gemv_workspace_bytes(const spax_matrix* W) {
  if (validate_matrix(W) != SPAX_OK) return 0;
  return gemv_ws(W);
}

int spax_tiered_gemv(const spax_matrix* W, const uint16_t* x, const int32_t* full_idx,
                     int32_t k_full, const int32_t* approx_idx, int32_t k_approx, uint16_t* y,
                     void* ws, size_t ws_bytes, hipStream_t stream, const spax_copy* copy) {
  int st = validate_product(W, x, full_idx, k_full, approx_idx, k_approx, ws, ws_bytes, copy);
  if (st) return st;
  if (!y) return SPAX_ENULL;
  if (!aligned16(y)) return SPAX_EALIGN;
  return run_product(W, x, full_idx, k_full, approx_idx, k_approx, kEpiPlain, y, nullptr,
                     nullptr, nullptr, ws, stream, copy);
}

size_t spax_layer_workspace_bytes(const spax_layer* L) {
  if (!L) return 0;
  size_t m = 0;
  bool any = false;
  for (int g = 0; g < 4; ++g)
    if (L->group[g].cols > 0 && validate_matrix(&L->group[g]) == SPAX_OK) {
      m = std::max(m, gemv_ws(&L->group[g]));
      any = true;
    }
  return any ? std::max(m, layer_ws(L)) : 0;
}

int spax_layer_step(const spax_layer* L, const spax_layer_io* io, void* ws, size_t ws_bytes,
                    hipStream_t compute_stream, const spax_copy* copy) {
  if (!L || !io) return SPAX_ENULL;
  const spax_matrix* G = L->group;
  if (L->kernel != SPAX_KERNEL_AUTO && L->kernel != SPAX_KERNEL_SEPARATE &&
      L->kernel != SPAX_KERNEL_PER_GROUP)
    return SPAX_EINVAL;
  if (L->workgroups < 0 || L->workgroups > kLayerMaxWgs) return SPAX_EINVAL;
  const bool has_gu = G[SPAX_GROUP_GATE_UP].cols > 0, has_dn = G[SPAX_GROUP_DOWN].cols > 0;
  if (has_gu && G[SPAX_GROUP_GATE_UP].layout != SPAX_LAYOUT_GLU_INTERLEAVED) return SPAX_EINVAL;
  if (has_dn && G[SPAX_GROUP_DOWN].layout != SPAX_LAYOUT_PLAIN) return SPAX_EINVAL;
  if (has_gu && has_dn && G[SPAX_GROUP_DOWN].cols != G[SPAX_GROUP_GATE_UP].rows / 2)
    return SPAX_EINVAL;
  const uint16_t* inputs[4] = {io->h, io->z, io->x, io->a};
  uint16_t* outputs[4] = {io->qkv, io->o, io->a, io->down};
  if (ws_bytes < spax_layer_workspace_bytes(L)) return SPAX_EWORKSPACE;
  // validate everything before enqueuing anything
  for (int g = 0; g < 4; ++g) {
    if (G[g].cols <= 0) continue;
    if (g != SPAX_GROUP_GATE_UP && G[g].layout != SPAX_LAYOUT_PLAIN) return SPAX_EINVAL;
    int st = validate_product(&G[g], inputs[g], io->full_idx[g], L->k_full[g],
                              io->approx_idx[g], L->k_approx[g], ws, ws_bytes, copy);
    if (st) return st;
    if (G[g].cols > 65536) return SPAX_EINVAL;
    if (!outputs[g]) return SPAX_ENULL;
    if (!aligned16(outputs[g]) || !aligned16(io->g) || !aligned16(io->u)) return SPAX_EALIGN;
  }
  int32_t ff = 0, af = 0;
  if (L->kernel == SPAX_KERNEL_AUTO && layer_fits(L, &ff, &af)) {
    LayerArgs A;
    bool ok = false;
    const int st = plan_layer_kernel(L, &A, &ok);
    if (st) return st;
    if (ok) return run_layer_kernel(L, io, ws, ff, af, A, compute_stream);
  }
  const bool separate = L->kernel == SPAX_KERNEL_SEPARATE;
  for (int g = 0; g < 4; ++g) {
    if (G[g].cols <= 0) continue;
    const int32_t kf = L->k_full[g], ka = L->k_approx[g];
    uint16_t* y = g == SPAX_GROUP_GATE_UP ? nullptr : outputs[g];
    uint16_t* ga = g == SPAX_GROUP_GATE_UP ? io->a : nullptr;
    uint16_t* gg = g == SPAX_GROUP_GATE_UP ? io->g : nullptr;
    uint16_t* gu = g == SPAX_GROUP_GATE_UP ? io->u : nullptr;
    const int32_t epi = g == SPAX_GROUP_GATE_UP ? kEpiGlu : kEpiPlain;
    ProductPlan fp;
    int st;
    if (!separate && G[g].cols > kRankMaxN && plan_piece(&G[g], kf, ka, &fp)) {
      // long input: the sliced selection finds the thresholds and slice
      // counts; every product workgroup places its own piece from them
      hipError_t e = launch_select(inputs[g], G[g].cols, kf, ka, nullptr, nullptr,
                                   select_scratch(ws), compute_stream);
      if (e != hipSuccess) return hip_fail(e);
      st = run_product(&G[g], inputs[g], nullptr, kf, nullptr, ka, epi, y, ga, gg, gu, ws,
                       compute_stream, copy, &fp, kListSliced, io->full_idx[g],
                       io->approx_idx[g]);
    } else if (!separate && G[g].cols > kRankMaxN) {
      // long input, host-resident weights: lists in memory for the copy
      hipError_t e = launch_select(inputs[g], G[g].cols, kf, ka, io->full_idx[g],
                                   io->approx_idx[g], select_scratch(ws), compute_stream);
      if (e != hipSuccess) return hip_fail(e);
      st = run_product(&G[g], inputs[g], io->full_idx[g], kf, io->approx_idx[g], ka, epi, y, ga,
                       gg, gu, ws, compute_stream, copy);
    } else if (!separate && plan_piece(&G[g], kf, ka, &fp)) {
      // device-resident weights: selection fused into the product
      st = run_product(&G[g], inputs[g], nullptr, kf, nullptr, ka, epi, y, ga, gg, gu, ws,
                       compute_stream, copy, &fp, kListRank, io->full_idx[g],
                       io->approx_idx[g]);
    } else {
      hipError_t e = launch_plan(inputs[g], G[g].cols, kf, ka, io->full_idx[g],
                                 io->approx_idx[g], compute_stream);
      if (e != hipSuccess) return hip_fail(e);
      st = run_product(&G[g], inputs[g], io->full_idx[g], kf, io->approx_idx[g], ka, epi, y, ga,
                       gg, gu, ws, compute_stream, copy);
    }
    if (st) return st;
  }
  return SPAX_OK;
}

int spax_layer_schedule(const spax_layer* L, int32_t workgroups, int32_t* out, int64_t cap,
                        int64_t* count) {
  if (!L || !count || (cap > 0 && !out)) return SPAX_ENULL;
  if (cap < 0 || workgroups < 0 || workgroups > kLayerMaxWgs) return SPAX_EINVAL;
  for (int g = 0; g < 4; ++g) {
    if (L->group[g].cols <= 0) continue;
    if (validate_matrix(&L->group[g]) != SPAX_OK) return SPAX_EINVAL;
    if (check_counts(L->group[g].cols, L->k_full[g], L->k_approx[g])) return SPAX_EINVAL;
  }
  int32_t ff = 0, af = 0;
  if (!layer_fits(L, &ff, &af)) return SPAX_EINVAL;
  int32_t G = workgroups;
  if (G == 0) {
    int32_t cus = 0;
    const int st = device_cus(&cus);
    if (st) return st;
    G = layer_workgroups(cus);
  }
  LayerArgs A;
  layer_schedule(L, G, &A);
  if (!layer_segs_fit(A)) return SPAX_EINVAL;
  int64_t n = 0;
  for (int32_t w = 0; w < A.G; ++w) {
    for (int oi = 0; oi < A.n_order; ++oi) {
      layer_group_segs(A, A.order[oi], (uint32_t)w, [&](const LayerSeg& s0) {
        LayerSeg s = s0;
        layer_contributors(A, s);
        if (n < cap) {
          int32_t* r = out + 9 * n;
          r[0] = w; r[1] = s.g; r[2] = s.t; r[3] = s.f0; r[4] = s.f1;
          r[5] = s.a0; r[6] = s.a1; r[7] = s.w_lo; r[8] = s.w_hi;
        }
        ++n;
      });
    }
  }
  *count = n;
  return SPAX_OK;
}

int spax_workspace_status(void* ws, hipStream_t stream, int32_t reset, uint32_t* status) {
  if (!ws || !status) return SPAX_ENULL;
  uint32_t* word = sync_words(ws) + 2;
  hipError_t e = hipMemcpyAsync(status, word, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && reset && *status) {
    const uint32_t zero = 0u;
    e = hipMemcpyAsync(word, &zero, sizeof(uint32_t), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

int spax_sq_error(const uint16_t* y, const uint16_t* ref, int64_t n, double* acc,
                  int32_t accumulate, hipStream_t stream) {
  if (!acc || (n > 0 && (!y || !ref))) return SPAX_ENULL;
  if (n < 0) return SPAX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(ref)) % 2 ||
      reinterpret_cast<uintptr_t>(acc) % 8)
    return SPAX_EALIGN;
  const hipError_t e = launch_sq_error(y, ref, n, acc, accumulate, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

int spax_pack_g128(const uint16_t* w, int32_t rows, int32_t cols, int32_t fmt, uint8_t* codes,
                   uint16_t* scales, hipStream_t stream) {
  if (fmt != kInt4 && fmt != kInt2) return SPAX_EFORMAT;
  if (rows <= 0 || cols <= 0 || rows % kGroup) return SPAX_EINVAL;
  if (!w || !codes || !scales) return SPAX_ENULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return SPAX_EALIGN;
  const hipError_t e = launch_pack(w, rows, cols, fmt, codes, scales, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

int spax_pack_sign2(const uint16_t* w, int32_t rows, int32_t cols, uint8_t* codes,
                    uint16_t* scales, hipStream_t stream) {
  if (!w || !codes || !scales) return SPAX_ENULL;
  if (rows <= 0 || cols <= 0 || rows % kGroup || rows > kMaxRows) return SPAX_EINVAL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return SPAX_EALIGN;
  const hipError_t e = launch_pack_sign2(w, rows, cols, codes, scales, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

size_t spax_pack_trellis_workspace_bytes(int32_t rows, int32_t batch) {
  if (rows <= 0 || batch <= 0) return 0;
  return (size_t)batch * trellis_ws_per_column(rows);
}

int spax_pack_trellis(const uint16_t* w, int32_t rows, int32_t cols, const uint16_t* codebook,
                      uint8_t* codes, uint16_t* scales, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!w || !codebook || !codes || !scales || !ws) return SPAX_ENULL;
  if (rows <= 0 || cols <= 0 || rows % kGroup || rows > kMaxRows) return SPAX_EINVAL;
  if (!aligned16(w) || !aligned16(codebook) || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(ws))
    return SPAX_EALIGN;
  if (ws_bytes < trellis_ws_per_column(rows)) return SPAX_EWORKSPACE;
  const hipError_t e =
      launch_pack_trellis(w, rows, cols, codebook, codes, scales, ws, ws_bytes, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

int spax_workspace_clear(void* ws, size_t bytes, hipStream_t stream) {
  if (bytes % 4) return SPAX_EINVAL;
  if (bytes == 0) return SPAX_OK;
  if (!ws) return SPAX_ENULL;
  if (!aligned16(ws)) return SPAX_EALIGN;
  const hipError_t e = launch_clear(ws, bytes, stream);
  return e == hipSuccess ? SPAX_OK : hip_fail(e);
}

}  // extern "C"
