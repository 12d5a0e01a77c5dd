/*
 * spax.h -- C ABI of the three-tier activation-sparse decode library (gfx950).
 *
 * Method: "Activation Sparsity with Weight Approximation for Faster LLM
 * Decoding on Offloaded Weights" (the SpAx page). For each token and each
 * projection the input activations are ranked by magnitude; the columns of
 * the smallest are skipped, the next ones are read from a compressed copy and
 * the largest ones are read in full precision (section 1; section 5,
 * Figure 2 steps 3-5), giving y = W[:,F] x_F + W^[:,A] x_A (section 2 Eq. 1
 * restricted to the kept columns).
 *
 * Conventions shared by every call
 *   - fp16 values travel as uint16_t bit patterns; indices are int32_t.
 *   - Matrices are column-major: column j of an R-row matrix is contiguous.
 *     One column per activation entry keeps a selected column readable on
 *     its own (section 1, challenge 1; section 5.1).
 *   - Group-128 codes: a group is 128 consecutive rows of one column with one
 *     fp16 scale, so each column is rebuilt from its own codes (section 5.1).
 *       int4: s = fp16(max|w| / 7), q = clamp(rne(w / s), -8, 7), w^ = q s;
 *             row 2i in bits 0-3 of byte i of the column, row 2i+1 in 4-7.
 *       int2: s = fp16(max|w| / 1.5), u = clamp(rne(w / s + 1.5), 0, 3),
 *             w^ = (u - 1.5) s  (the sign-pair form of section 5.1 Eq. 4
 *             with scales s and s/2); row 4i+r in bits 2r..2r+1 of byte i.
 *       codes: [cols][rows/2] (int4) or [cols][rows/4] (int2) bytes;
 *       scales: [cols][rows/128] fp16.
 *   - rows must be a multiple of 128 for every format and at most
 *     SPAX_MAX_ROWS.
 *   - Every device pointer must be 16-byte aligned.
 *   - The caller owns every buffer. Calls validate their arguments on the
 *     host, enqueue kernels on the given stream(s) and return; results are
 *     valid once the stream has reached that point. No call allocates memory.
 *   - A status code is returned; 0 is success. Validation errors return
 *     before anything is enqueued. No exception crosses the ABI.
 */
#ifndef SPAX_H_
#define SPAX_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define SPAX_OK          0
#define SPAX_EINVAL     -1  /* a size or a tier count is out of range          */
#define SPAX_ENULL      -2  /* a required pointer is null                      */
#define SPAX_EALIGN     -3  /* a device pointer is not 16-byte aligned         */
#define SPAX_EFORMAT    -4  /* unknown format or unsupported combination       */
/* Largest matrix height (rows) the product accepts. */
#define SPAX_MAX_ROWS 1048576
#define SPAX_EWORKSPACE -5  /* workspace smaller than the *_workspace_bytes()  */
#define SPAX_ESTREAM    -6  /* host-resident matrix without a spax_copy set up
                               on the current device                           */
#define SPAX_EHIP       -7  /* the HIP runtime reported an error; see
                               spax_last_error()                               */
#define SPAX_ENOMEM     -8  /* host memory for scratch could not be allocated
                               (spax_pack_trellis_host)                        */

/* ---- formats, residency, layout ---------------------------------------- */
#define SPAX_FMT_NONE       0  /* tier absent (its count must be 0)          */
#define SPAX_FMT_FP16       1  /* fp16 values, rows*2 bytes per column        */
#define SPAX_FMT_INT4_G128  2  /* int4 codes + fp16 scale per 128 rows        */
#define SPAX_FMT_INT2_G128  3  /* int2 codes + fp16 scale per 128 rows        */
/* Two-scale 2-bit sign code of the middle tier (SpAx page section 5.1,
 * Eq. 4): weight i of column j is rebuilt as e1 s_{j,0} + e2 s_{j,1} with
 * signs (e1, e2) in {-1, +1} and two fp16 scales per matrix column. Code u
 * = 2 [e1 = -1] + [e2 = -1], rows/4 bytes per column packed like int2 (row
 * 4i + r in bits 2r..2r+1 of byte i); scales [cols][S][2] = (s0, s1) of each
 * of the S matrices a stored column holds (spax_matrix.approx_seg_rows).
 * Approx tier only, with an fp16 full tier. Produced by spax_pack_sign2 per
 * matrix. */
#define SPAX_FMT_SIGN2      4
/* Trellis-coded middle tier (SpAx page section 5.1, trellis coding): 2-bit
 * codes, rows/4 bytes per column in the int2 packing, one fp16 scale per
 * matrix column (scales [cols][S], S matrices per stored column, see
 * spax_matrix.approx_seg_rows), and a shared fp16 codebook of 65536 values
 * (spax_matrix.approx_codebook, device memory). Weight i of a column is
 * codebook[index_i] * scale, index_i = (index_{i-1} >> 2) | (c_i << 14),
 * index_{-1} = 0. Approx tier only, with an fp16 full tier. The product
 * keeps the codebook in LDS (its fused ranking then holds list pieces of at
 * most 1024 positions). Produced by spax_pack_trellis (GPU) or
 * spax_pack_trellis_host (host), which give the same bits. */
#define SPAX_FMT_TRELLIS    5

#define SPAX_RES_DEVICE       0  /* weights in device memory (HBM)            */
#define SPAX_RES_HOST_PINNED  1  /* weights in pinned host memory that the GPU
                                    can address (hipHostMalloc); only the
                                    selected columns cross the host link       */

#define SPAX_LAYOUT_PLAIN           0
/* Gate and up projections of a gated FFN (section 2: a = silu(W_gate x) *
 * W_up x) stored as ONE matrix of 2*I rows whose column j holds the two
 * column-j segments interleaved in 128-row blocks:
 *   stored rows [256b, 256b+128)     = gate rows [128b, 128b+128)
 *   stored rows [256b+128, 256b+256) = up   rows [128b, 128b+128)
 * The two matrices share one ranking and one request per entry (section 5.3,
 * Figure 4: the columns that one activation entry indexes are adjacent). */
#define SPAX_LAYOUT_GLU_INTERLEAVED 1

/* One projection (or one group of projections stacked row-wise). */
typedef struct spax_matrix {
  int32_t rows;            /* output length R (multiple of 128)            */
  int32_t cols;            /* input length n                                */
  int32_t full_fmt;        /* SPAX_FMT_FP16 or SPAX_FMT_INT4_G128           */
  int32_t approx_fmt;      /* SPAX_FMT_NONE, _INT4_G128, _INT2_G128, _SIGN2
                              or _TRELLIS (the last two with an fp16 full
                              tier)                                         */
  int32_t residency;       /* SPAX_RES_*                                    */
  int32_t layout;          /* SPAX_LAYOUT_*                                 */
  int32_t approx_seg_rows; /* SIGN2 / TRELLIS approx tiers: a stored column
                              holding several matrices' columns (q, k, v
                              stacked) has rows / approx_seg_rows segments
                              of approx_seg_rows rows (a multiple of 512
                              dividing rows), each coded as its own matrix
                              column (SpAx page section 5.1: codes and
                              scales per weight column; section 5.3 Figure
                              4: stacked columns stay distinct columns).
                              0: one matrix. GLU_INTERLEAVED always holds two
                              matrices, gate and up. Ignored by the other
                              formats (their scales are per 128 rows).     */
  const void* full_data;   /* fp16 [cols][rows] or int4 codes [cols][rows/2] */
  const uint16_t* full_scales;   /* int4 full tier only: [cols][rows/128]   */
  const uint8_t* approx_codes;   /* approx codes, layout per approx_fmt     */
  const uint16_t* approx_scales; /* [cols][rows/128]; SIGN2: [cols][S][2];
                                    TRELLIS: [cols][S], S the matrices per
                                    stored column (segment s first)         */
  const uint16_t* approx_codebook; /* TRELLIS only: device fp16 [65536]     */
} spax_matrix;

/* ---- host-resident copies ---------------------------------------------- */
/* The stream and events a host-resident product uses to copy the selected
 * columns into device staging while the product consumes earlier chunks
 * (section 5, Figure 2 step 4). spax_copy_init creates the events on the
 * current device once; the per-token calls only record and wait on them.
 * spax_copy_release destroys them. The caller owns the stream.
 *   Errors: SPAX_ENULL, SPAX_EHIP.                                           */
#define SPAX_COPY_CHUNKS 4
typedef struct spax_copy {
  hipStream_t stream;                    /* the copy stream (caller's)       */
  hipEvent_t ready;                      /* lists ready on the compute stream */
  hipEvent_t chunk[SPAX_COPY_CHUNKS];    /* chunk k landed in staging        */
  int32_t device;                        /* device the events belong to      */
} spax_copy;

int spax_copy_init(spax_copy* copy, hipStream_t copy_stream);
int spax_copy_release(spax_copy* copy);

/* ---- tier selection ----------------------------------------------------- */
/* spax_plan_tiers -- rank x by magnitude and split its entries into tiers.
 *   SpAx page section 2 (magnitude top-k keeps the largest |x_i|) and
 *   section 5, Figure 2 step 3 with section 5.2 (a second boundary divides
 *   the kept entries; k_top and k_mid are integers per group).
 *   x          device, fp16[n], 16-byte aligned; read only.
 *   n          1 .. 65536.
 *   k_full     number of full-tier entries (k_top), >= 0.
 *   k_approx   number of middle-tier entries (k_mid), >= 0, k_full+k_approx <= n.
 *   full_idx   device int32[k_full]   out: ascending indices of the k_full
 *              largest |x_j|.
 *   approx_idx device int32[k_approx] out: ascending indices of the next
 *              k_approx.
 *   Ties in |x| rank the lower index first; +0 and -0 are equal; the order
 *   key is the fp16 magnitude bit pattern (inf above every finite value).
 *   The result is deterministic and bit-exact.
 *   Errors: SPAX_ENULL, SPAX_EINVAL (sizes), SPAX_EALIGN, SPAX_EHIP.       */
int spax_plan_tiers(const uint16_t* x, int32_t n, int32_t k_full, int32_t k_approx,
                    int32_t* full_idx, int32_t* approx_idx, hipStream_t stream);

/* ---- tiered product ----------------------------------------------------- */
/* Workspace bytes one spax_tiered_gemv call on W needs (any tier counts). */
size_t spax_gemv_workspace_bytes(const spax_matrix* W);

/* spax_tiered_gemv -- y = sum_{j in F} x_j W~[:,j] + sum_{j in A} x_j W^[:,j].
 *   SpAx page section 2 Eq. 1 and section 5, Figure 2 steps 4-5: the full
 *   tier is read in its stored format (fp16, or int4 dequantised), the middle
 *   tier is rebuilt from its codes on the GPU, the skipped columns are never
 *   read. Products and sums in fp32, y rounded once to fp16 (nearest even).
 *   W          matrix descriptor (host struct, read during the call only).
 *   x          device fp16[W->cols].
 *   full_idx   device int32[k_full], approx_idx device int32[k_approx]:
 *              in-range, disjoint; any order is accepted, the fp32 summation
 *              follows list order.
 *   y          device fp16[W->rows] out (stored row order; for the
 *              GLU-interleaved layout this is the interleaved order).
 *   ws         device workspace of spax_gemv_workspace_bytes(W) bytes. It
 *              must be all zero before its first use (spax_workspace_clear);
 *              every call leaves its counters at zero again. The counters
 *              and the selection scratch sit at fixed places at the start of
 *              every workspace, so one workspace (sized for the largest
 *              matrix) may serve any mix of matrices and calls. Calls that
 *              share a workspace must be ordered on one stream.
 *   stream     compute stream. copy: required when W is
 *              SPAX_RES_HOST_PINNED (a spax_copy set up by spax_copy_init on
 *              this device: only the selected columns are copied to device
 *              staging inside ws, in chunks overlapped with the product),
 *              ignored otherwise (may be null).
 *   k_full = k_approx = 0 writes zeros. The result is deterministic: the
 *   same inputs give the same bits, in both residency modes.
 *   Errors: SPAX_ENULL, SPAX_EINVAL, SPAX_EALIGN, SPAX_EFORMAT,
 *   SPAX_EWORKSPACE, SPAX_ESTREAM (host-resident W without a copy set up on
 *   this device), SPAX_EHIP.                                                 */
int spax_tiered_gemv(const spax_matrix* W, const uint16_t* x,
                     const int32_t* full_idx, int32_t k_full,
                     const int32_t* approx_idx, int32_t k_approx,
                     uint16_t* y, void* ws, size_t ws_bytes,
                     hipStream_t stream, const spax_copy* copy);

/* ---- one decoder layer -------------------------------------------------- */
#define SPAX_GROUP_QKV     0  /* W_q, W_k, W_v stacked row-wise; input h   */
#define SPAX_GROUP_O       1  /* W_o; input z                               */
#define SPAX_GROUP_GATE_UP 2  /* W_gate, W_up, GLU-interleaved; input x     */
#define SPAX_GROUP_DOWN    3  /* W_down; input a = silu(g) * u              */

/* The seven matrices of a layer in the four groups that share a ranking
 * (section 2; section 5.2 step 1; section 5.3 Figure 4). A group whose
 * matrix has cols == 0 is absent and skipped. GATE_UP must use
 * SPAX_LAYOUT_GLU_INTERLEAVED; with both present, DOWN must have
 * cols == GATE_UP.rows / 2 and reads the a that GATE_UP writes. DOWN alone
 * reads a caller-provided a (io->a). */
/* How spax_layer_step runs the groups (per call, field spax_layer.kernel):
 *   SPAX_KERNEL_AUTO       one launch for the whole layer (the layer kernel:
 *                          persistent workgroups, one per compute unit, whose
 *                          ranking waves rank each group's input in LDS while
 *                          the streaming waves read the previous group's
 *                          columns) when every present group is
 *                          device-resident, all groups share one format pair
 *                          other than the trellis code, every input is at most
 *                          32768 long and the groups' lists fit its LDS
 *                          (24576 positions in all); otherwise as
 *                          SPAX_KERNEL_PER_GROUP;
 *   SPAX_KERNEL_SEPARATE   per group, the stand-alone selection kernel, then
 *                          the tiered product reading the lists from memory;
 *   SPAX_KERNEL_PER_GROUP  per group, one launch whose workgroups each rank
 *                          the input in LDS (inputs up to 32768 long; longer
 *                          ones are ranked by three short launches over
 *                          4096-entry slices first) where the list pieces fit,
 *                          else as SPAX_KERNEL_SEPARATE. Host-resident groups
 *                          always take the stand-alone selection and the
 *                          staged copy.
 * All compute the same lists; the products agree within the error bound of
 * spax_tiered_gemv. Each choice is deterministic; SEPARATE and PER_GROUP
 * add the partial sums in the same order (and host-resident groups give the
 * same bits as device-resident ones under them), the layer kernel cuts the
 * columns differently and so may differ from them in the last bits. */
#define SPAX_KERNEL_AUTO      0
#define SPAX_KERNEL_SEPARATE  1
#define SPAX_KERNEL_PER_GROUP 2

typedef struct spax_layer {
  spax_matrix group[4];
  int32_t k_full[4];
  int32_t k_approx[4];
  int32_t kernel;          /* SPAX_KERNEL_*                                 */
  int32_t workgroups;      /* layer kernel: most workgroups of the launch;
                            * 0 = one per compute unit. At most 512 and
                            * never more than the device's compute units
                            * (larger values are cut to that: the launch
                            * needs all of its workgroups resident).      */
} spax_layer;

/* Inputs, outputs and per-group tier lists (all device pointers). */
typedef struct spax_layer_io {
  const uint16_t* h;       /* fp16[QKV.cols]                                 */
  const uint16_t* z;       /* fp16[O.cols]                                   */
  const uint16_t* x;       /* fp16[GATE_UP.cols]                             */
  uint16_t* qkv;           /* out fp16[QKV.rows] (q, k, v in stored order)   */
  uint16_t* o;             /* out fp16[O.rows]                               */
  uint16_t* g;             /* out fp16[I] gate output, may be null           */
  uint16_t* u;             /* out fp16[I] up output, may be null             */
  uint16_t* a;             /* out fp16[I] = fp16(silu(g) * u)                */
  uint16_t* down;          /* out fp16[DOWN.rows]                            */
  int32_t* full_idx[4];    /* out per group, int32[k_full[g]]                */
  int32_t* approx_idx[4];  /* out per group, int32[k_approx[g]]              */
} spax_layer_io;

size_t spax_layer_workspace_bytes(const spax_layer* L);

/* spax_layer_step -- rank each group's input once, then run the group's
 * tiered product with the shared lists: h -> q,k,v; z -> o; x -> gate,up;
 * a = silu(g) * u is formed in the gate/up product's final reduction (fp32
 * math on the fp16 g and u, one rounding); a -> down.
 *   SpAx page section 2 (matrices and inputs), sections 5.2-5.3 (groups).
 *   ws / ws_bytes as for spax_tiered_gemv, sized by
 *   spax_layer_workspace_bytes(L). copy is required when any group is
 *   host-resident. L->kernel picks the launch form (SPAX_KERNEL_*).
 *   The layer kernel waits, inside the launch, for the gate/up tiles before
 *   ranking a; it assumes its workgroups (one per compute unit) run at the
 *   same time, i.e. no other work holds compute units for long while it
 *   runs. Its waits are bounded: one that runs out sets a bit of the
 *   workspace status (spax_workspace_status) and the results of that call
 *   are not valid. Deterministic.
 *   Errors: as spax_tiered_gemv; SPAX_EINVAL for an unknown L->kernel or
 *   L->workgroups outside [0, 512].                                          */
int spax_layer_step(const spax_layer* L, const spax_layer_io* io,
                    void* ws, size_t ws_bytes,
                    hipStream_t compute_stream, const spax_copy* copy);

/* spax_layer_step_static -- spax_layer_step without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). It allocates
 * nothing: its scratch (arrival counters, sync words, partial sums) is one
 * static 16 MiB device array per GPU, held by the library until the process
 * ends. Device-resident weights only (no copy context).
 *   L, io, stream  as for spax_layer_step.
 *   Every call on one GPU uses that GPU's array: its counters are cleared at
 *   the start of each call (a fill kernel on `stream`), so calls on one GPU
 *   must not overlap (one stream, or ordered streams); overlapping calls
 *   race on the array.
 *   Errors: as spax_layer_step; SPAX_EWORKSPACE (message in
 *   spax_last_error) when spax_layer_workspace_bytes(L) exceeds 16 MiB,
 *   checked before any GPU call.                                           */
int spax_layer_step_static(const spax_layer* L, const spax_layer_io* io,
                           hipStream_t stream);

/* spax_layer_schedule -- the layer kernel's work schedule, for inspection
 * (host only, enqueues nothing). For every workgroup w of `workgroups`
 * (0: the number the library would launch on the current device) and every
 * piece of work in processing order, 9 int32 values: w, group id (SPAX_GROUP_*),
 * row tile, first and end full-tier list positions, first and end
 * approx-tier list positions, and the first and last workgroup that work on
 * the same tile. Tile t covers stored rows [512 t, 512 t + 512); a
 * workgroup's positions of a tile index the ascending tier lists of the
 * group. Writes at most `cap` records to `out` (may be null with cap 0) and
 * the total number of records to *count.
 *   Errors: SPAX_ENULL, SPAX_EINVAL (the layer kernel does not apply to L,
 *   a workgroup would meet more than 160 row tiles in one phase, or
 *   workgroups out of range), SPAX_EHIP (workgroups 0 without a device).   */
int spax_layer_schedule(const spax_layer* L, int32_t workgroups, int32_t* out, int64_t cap,
                        int64_t* count);

/* spax_workspace_status -- the sticky status bits the layer kernel leaves in
 * a workspace (0: none; bit 0: an LDS wait ran out, bit 1: the wait for the
 * gate/up tiles ran out). Copies 4 bytes to the host and synchronises the
 * stream. reset != 0 also clears the bits.
 *   Errors: SPAX_ENULL, SPAX_EHIP.                                           */
int spax_workspace_status(void* ws, hipStream_t stream, int32_t reset, uint32_t* status);

/* ---- offline helpers ---------------------------------------------------- */
/* spax_sq_error -- the squared l2 distance of two fp16 vectors, for the
 * offline calibration of the tier sizes (SpAx page section 5.2, steps 1-2:
 * the tier sizes that keep the layer's l2 output error against the dense
 * product smallest): sum_i (y_i - ref_i)^2, each difference and square formed
 * in fp64, stored to *acc (accumulate == 0) or added to it (accumulate != 0).
 * One workgroup in a fixed order: repeated calls give the same bits. Several
 * calls on one stream (one per calibration token) need one synchronisation
 * before *acc is read.
 *   y, ref  device fp16 [n] (2-byte aligned; may be null when n == 0);
 *   acc  device fp64 (8-byte aligned), read and written by the kernel;
 *   n >= 0 (0 sums nothing: *acc is set to 0 or kept).
 *   Errors: SPAX_ENULL, SPAX_EINVAL (n < 0), SPAX_EALIGN, SPAX_EHIP.        */
int spax_sq_error(const uint16_t* y, const uint16_t* ref, int64_t n, double* acc,
                  int32_t accumulate, hipStream_t stream);

/* spax_pack_g128 -- encode the compressed copy of a matrix (SpAx page
 * section 5, Figure 2 step 1: every column is encoded offline, on its own).
 *   w      device fp16 [cols][rows] (column-major), rows % 128 == 0.
 *   fmt    SPAX_FMT_INT4_G128 or SPAX_FMT_INT2_G128.
 *   codes  device out, [cols][rows/2] or [cols][rows/4] bytes.
 *   scales device out, fp16 [cols][rows/128].
 *   Bit-exact to the rules in the header comment above.
 *   Errors: SPAX_ENULL, SPAX_EINVAL, SPAX_EALIGN, SPAX_EFORMAT, SPAX_EHIP.  */
int spax_pack_g128(const uint16_t* w, int32_t rows, int32_t cols, int32_t fmt,
                   uint8_t* codes, uint16_t* scales, hipStream_t stream);

/* spax_pack_sign2 -- encode the two-scale 2-bit sign code of a matrix
 * (SpAx page section 5.1, Eq. 4; offline, Figure 2 step 1). Per column j,
 * with every weight taken exactly (units of 2^-24):
 *   s0 = fp16(mean_i |w_i|)                 (the least-squares scale of the
 *   s1 = fp16(mean_i |w_i - e1_i s0|)        sign code e1_i = +1 iff w_i >= 0,
 *                                            then of the residual's sign)
 *   (e1, e2) = argmin over {-1,+1}^2 of (w_i - e1 s0 - e2 s1)^2, the smaller
 *   code u on equal errors.
 * The sums are exact; each mean is one fp64 division rounded once to fp16
 * (ties to even). The page fits its scales Lloyd-Max style; this closed
 * form is the reading taken where its fitting text is not available.
 *   w      device fp16 [cols][rows] (column-major), finite, rows % 128 == 0.
 *   codes  device out, [cols][rows/4] bytes.
 *   scales device out, fp16 [cols][2] = (s0, s1).
 *   Errors: SPAX_ENULL, SPAX_EINVAL, SPAX_EALIGN, SPAX_EHIP.                */
int spax_pack_sign2(const uint16_t* w, int32_t rows, int32_t cols, uint8_t* codes,
                    uint16_t* scales, hipStream_t stream);

/* spax_pack_trellis_host -- encode the trellis-coded middle tier of a matrix
 * (SpAx page section 5.1, trellis coding; offline, on the host, Figure 2
 * step 1). Per column: 2-bit codes c_i and one scale s, the column's
 * root-mean-square; weight i is rebuilt as codebook[index_i] * s with
 * index_i = (index_{i-1} >> 2) | (c_i << 14), index_{-1} = 0 (the window of
 * the codes of rows i-7..i, the oldest in the low bits). The codes minimise
 * sum_i (w_i / s - codebook[index_i])^2 (Viterbi over the 2^14 states of the
 * last seven codes), with the arithmetic fixed operation by operation:
 *   s = fp16(sqrt(fp64(fp64(S) / rows)) 2^-24), S = sum w_i^2 exactly;
 *   v_i = fp32(w_i / s); per candidate d = v_i - cb, e = d * d, cost + e in
 *   fp32; ties keep the smallest dropped code, then the smallest final state.
 * A zero column gets s = 0 and zero codes.
 *   w        host fp16 [cols][rows] (column-major), finite, rows % 128 == 0.
 *   codebook host fp16 [65536] (values the caller drew once, e.g. N(0, 1)).
 *   codes    host out, [cols][rows/4] bytes, row 4i + r in bits 2r..2r+1 of
 *            byte i.
 *   scales   host out, fp16 [cols].
 *   threads  host threads to use (columns are independent), >= 1.
 *   Memory: about rows * 16 KB of host scratch per thread, allocated before
 *   any thread starts; when only some threads' scratch fits, fewer threads
 *   run (and fewer again if a thread cannot be started).
 *   Errors: SPAX_ENULL, SPAX_EINVAL; SPAX_ENOMEM when not even one thread's
 *   scratch can be allocated (codes and scales are then left unwritten).     */
int spax_pack_trellis_host(const uint16_t* w, int32_t rows, int32_t cols,
                           const uint16_t* codebook, uint8_t* codes, uint16_t* scales,
                           int32_t threads);

/* spax_pack_trellis -- the same encoding as spax_pack_trellis_host, on the
 * GPU (every code and scale bit-identical): one 1024-thread workgroup per
 * column runs the 16384-state Viterbi, two barriers' worth of work per row,
 * and traces the best path back from backpointers kept in the workspace.
 *   w, codebook, codes, scales  device memory, layouts as in
 *            spax_pack_trellis_host; 16-byte aligned.
 *   ws       device workspace of ws_bytes >= spax_pack_trellis_workspace_bytes(
 *            rows, 1); columns are encoded in launches of
 *            ws_bytes / spax_pack_trellis_workspace_bytes(rows, 1) columns.
 *   Enqueues only; results are valid after the stream synchronises.
 *   Errors: SPAX_ENULL, SPAX_EINVAL, SPAX_EALIGN, SPAX_EWORKSPACE, SPAX_EHIP. */
size_t spax_pack_trellis_workspace_bytes(int32_t rows, int32_t batch);
int spax_pack_trellis(const uint16_t* w, int32_t rows, int32_t cols, const uint16_t* codebook,
                      uint8_t* codes, uint16_t* scales, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* spax_workspace_clear -- zero `bytes` bytes of ws with a kernel (no memset
 * node, so it may be captured in a graph). bytes % 4 == 0. */
int spax_workspace_clear(void* ws, size_t bytes, hipStream_t stream);

/* Text for a status code (static storage). */
const char* spax_status_string(int status);

/* Text of the last HIP error seen by this thread (static per thread). */
const char* spax_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int spax_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* SPAX_H_ */
