/*
 * aq.h -- C ABI of the tile-aligned W4/W8 x A8 mixed-precision linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "AlignQuant: Tile-Aligned Mixed-Precision Quantization for
 * Efficient LLM Generation" (arXiv 2610.07457).  A projection Y = X W^T,
 * X in R^{M x K} (activation rows), W in R^{N x K} (rows = output features),
 * is cut into equal b_N x b_K weight tiles (Sec. 3.1).  Each tile stores one
 * representation, INT4 or INT8, selected by a 1-bit label (Sec. 3.2); the
 * runtime quantizes activations to INT8, widens every weight tile to INT8 on
 * chip, forms INT32 tile products and rescales them into an FP32 result
 * (Sec. 3.3; App. E.3 eq. 19).
 *
 * Conventions shared by every entry point
 *  - Pointers documented "device" are GPU global-memory pointers owned by the
 *    caller; "host" pointers are CPU memory owned by the caller.  The library
 *    never allocates, frees or retains caller memory and keeps no mutable
 *    global state; calls are re-entrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device work is enqueued asynchronously on it; results are ready when
 *    that stream is synchronized.  A fault inside a kernel surfaces at the
 *    caller's next synchronization, not as a return code.
 *  - All arguments are validated on the host before anything is enqueued; on
 *    any error nothing is launched and a negative aq_status is returned.  No
 *    C++ exception crosses this boundary.
 *  - GPU tile geometry: b_N = 64 and b_K in {64, 128}.  N % b_N == 0,
 *    K % b_K == 0.  Device buffers must be 16-byte aligned.
 *  - Inputs must be finite; NaN / Inf behaviour is unspecified.
 *
 * Packed layout (App. E.1-E.2; intra-tile order is this library's own, the
 * pages' CUTLASS order being specific to NVIDIA tensor cores)
 *  - labels  : ceil(R*C/8) bytes; tile t = r*C + j is bit (t & 7) of byte
 *              t >> 3 (first label in the least significant bit); 1 = INT4.
 *              The device buffer is padded with zero bytes to a whole number
 *              of 32-bit words (aq_plan.labels_alloc) so kernels read words.
 *  - row_off4, row_off8 : INT32[R+1]; number of INT4 (INT8) tiles in tile
 *              rows before r.  Tile (r, j) of precision b sits at
 *              index_b(r, j) = row_off_b[r] + (tiles of precision b before
 *              column j in row r)   (App. E.1 eq. 16).
 *  - w8      : T8 tiles of b_N*b_K bytes.  A tile is b_K/16 panels; panel p
 *              holds, for tile rows i = 0..b_N-1 in order, the 16 INT8 codes
 *              of columns 16p .. 16p+15.
 *  - w4      : T4 tiles of b_N*b_K/2 bytes.  A tile is b_K/32 panels; panel p
 *              holds, for tile rows i in order, 16 bytes; byte b packs the
 *              codes q0 at column 32p+b and q1 at column 32p+16+b as
 *              (q0 mod 16) + 16*(q1 mod 16)   (App. E.1 eq. 17).
 *  - s8, s4  : FP32[T_b][b_N]; the scale of row i of the tile at index_b(r,j)
 *              (one scale per tile row of each tile; the pages store one per
 *              tile, App. E.2).
 */
#ifndef AQ_H
#define AQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AQ_ABI_VERSION 11

typedef enum aq_status {
  AQ_OK = 0,
  AQ_ERR_NULL = -1,       /* a required pointer is NULL                      */
  AQ_ERR_SHAPE = -2,      /* N, K, M not compatible with the tile geometry   */
  AQ_ERR_TILE = -3,       /* tile size not supported on the GPU              */
  AQ_ERR_MAP = -4,        /* labels disagree with T4 / T8, or bad map entry  */
  AQ_ERR_ALIGN = -5,      /* a device pointer is not 16-byte aligned         */
  AQ_ERR_WORKSPACE = -6,  /* workspace missing or smaller than required      */
  AQ_ERR_HIP = -7,        /* the HIP runtime reported an error at launch     */
  AQ_ERR_ARG = -8         /* any other invalid argument                      */
} aq_status;

/* Sizes of a packed projection, computed on the host from its labels. */
typedef struct aq_plan {
  int32_t N, K, bN, bK;   /* projection and tile geometry                    */
  int32_t R, C;           /* tile rows N/bN and tile columns K/bK            */
  int32_t T4, T8;         /* INT4 and INT8 tile counts, T4 + T8 = R*C        */
  size_t labels_bytes;    /* ceil(R*C/8): the label bytes of App. E.2        */
  size_t labels_alloc;    /* 4*ceil(R*C/32): device allocation of the labels,
                             padded to whole 32-bit words (padding is zero)  */
  size_t offs_bytes;      /* 4*(R+1), for each of row_off4 and row_off8      */
  size_t w4_bytes, w8_bytes;  /* T4*bN*bK/2 and T8*bN*bK                     */
  size_t s4_bytes, s8_bytes;  /* 4*T4*bN and 4*T8*bN                         */
  size_t meta_bytes;      /* 24*R when C <= 128, else 0: host metadata image */
} aq_plan;

/* A packed projection: geometry plus device buffers sized by aq_plan.
 * aq_pack_weights writes the buffers; the linear entry points only read
 * them.  w4/s4 may be NULL when T4 == 0, w8/s8 when T8 == 0.
 * meta_host (optional, host memory, meta_bytes, 4-byte aligned, NULL if
 * unused): aq_pack_weights fills it with a host copy of the metadata, one
 * record of six 32-bit words per tile row r: row_off4[r], row_off8[r], then
 * the labels of tiles (r, 0 .. C-1) as 128 bits, LSB first (zero beyond C).
 * While it is set and the image is at most 3584 bytes (R <= 149),
 * aq_linear_decode passes it inside the kernel arguments, so no workgroup
 * waits on a metadata load before its first weight loads.  It must stay
 * valid and unchanged while decode calls are issued. */
typedef struct aq_packed {
  int32_t N, K, bN, bK, T4, T8;
  uint8_t *labels;        /* device, labels_alloc (4-byte aligned)          */
  int32_t *row_off4;      /* device, R+1                                    */
  int32_t *row_off8;      /* device, R+1                                    */
  uint8_t *w4;            /* device, w4_bytes                               */
  int8_t *w8;             /* device, w8_bytes                               */
  float *s4;              /* device, T4*bN                                  */
  float *s8;              /* device, T8*bN                                  */
  uint32_t *meta_host;    /* host, meta_bytes, optional                     */
} aq_packed;

/* Phase selector for aq_workspace_bytes / aq_linear_tile_partials;
 * AQ_PHASE_PREFILL_GROUPED sizes the workspace of aq_linear_prefill_grouped
 * and aq_linear_tile_partials_grouped, AQ_PHASE_DECODE_TRANSFORMED that of
 * aq_linear_decode_transformed, AQ_PHASE_DECODE_FP32 that of
 * aq_linear_decode_fp32 (workspace sizes only). */
#define AQ_PHASE_DECODE 0
#define AQ_PHASE_PREFILL 1
#define AQ_PHASE_PREFILL_GROUPED 2
#define AQ_PHASE_DECODE_TRANSFORMED 3
#define AQ_PHASE_DECODE_FP32 4

/* ABI version of the loaded library (AQ_ABI_VERSION). */
int aq_abi_version(void);

/* Human-readable text of a status code.  Never NULL. */
const char *aq_status_string(aq_status status);

/* Host only.  Labels from a precision map: zmap_host holds R*C entries in
 * row-major tile order, each 4 or 8 (Sec. 3.1 map z_{r,j}); labels_host
 * receives ceil(R*C/8) bytes, bit set = INT4, first tile in the LSB
 * (App. E.1).  AQ_ERR_MAP if an entry is neither 4 nor 8. */
aq_status aq_labels_from_map(const uint8_t *zmap_host, int R, int C, uint8_t *labels_host);

/* Host only.  Buffer sizes of a packed projection (App. E.2): checks the
 * geometry (any b_N >= 1 and b_K a multiple of 32 are planned; the GPU entry
 * points further require b_N = 64, b_K in {64, 128}) and counts T4 / T8 from
 * the host labels.  Does not touch the GPU. */
aq_status aq_plan_pack(int N, int K, int bN, int bK, const uint8_t *labels_host, aq_plan *out);

/* Quantize and pack one projection (App. B.2 eq. 5 with the 1e-12 floor of
 * eq. 6; App. E.1-E.2).  For tile (r, j) of precision b = 8 - 4*label and each
 * row n of it, s = max(max|W[n, tile cols]| / (2^(b-1) - 1), 1e-12) in FP64,
 * codes = clip(round_half_even(W / s), -2^(b-1), 2^(b-1) - 1) in FP64, the
 * stored scale is FP32(s) rounded to nearest even.
 *   W           device, FP32 [N][K] row-major; may be freed once the stream
 *               has passed this call.
 *   labels_host host, ceil(R*C/8) bytes; T4 / T8 in *out must match them.
 *   out         geometry (N, K, bN, bK, T4, T8) and device buffers, sized by
 *               aq_plan_pack.  labels (zero-padded to labels_alloc) and row
 *               offsets are copied in from the host; this call synchronizes
 *               `stream` once after those copies, so the host copy may be
 *               reused when it returns.  out->meta_host, when set, receives
 *               the host metadata image (see aq_packed).
 */
aq_status aq_pack_weights(const float *W, const uint8_t *labels_host, aq_packed *out, void *stream);

/* aq_pack_weights with the fitted scale of App. B.2 eq. 7 in place of the
 * absmax scale: for each tile row segment A (one output row, b_K columns) of
 * precision b, with s0 = max(max(0, max A) / (2^(b-1) - 1),
 * max(0, -min A) / 2^(b-1), 1e-12) (eq. 6), the scale is the first of
 * s_i = max((1/4 + i/128) s0, 1e-12), i = 0 .. 128, minimizing
 * sum_k (A_k - s_i Q_b(A_k; s_i))^2; FP64, the sum taken in column order
 * with each product and sum rounded on its own.  Codes Q_b(A; s), stored
 * scale FP32(s).  Arguments, layout and errors as aq_pack_weights; the
 * packed format is the same, so every linear entry point reads it. */
aq_status aq_pack_weights_mse(const float *W, const uint8_t *labels_host, aq_packed *out, void *stream);

/* Per-token INT8 activation quantization (App. B.3 FP64 preparation, eq. 5
 * rounding): for each row m, s = max(max_k |X[m,k]| / 127, 1e-12) in FP64,
 * qx[m,k] = clip(round_half_even(X[m,k] / s), -128, 127) in FP64,
 * sx[m] = FP32(s).
 *   X   device, FP32 [M][K] row-major;  qx device, INT8 [M][K];
 *   sx  device, FP32 [M].  K must be a multiple of 64; M == 0 is a no-op. */
aq_status aq_quant_act(const float *X, int M, int K, int8_t *qx, float *sx, void *stream);

/* Device workspace, in bytes, that aq_linear_decode (phase 0) or
 * aq_linear_prefill / aq_linear_tile_partials with phase 1 need for M rows
 * with the given decode split (0 = adaptive).  0 means no workspace is
 * needed.  The caller owns the workspace (16-byte aligned).
 *   Decode needs one when the call divides each row block's input columns
 *   into Z > 1 workgroup chunks (App. E.3 split-K across workgroups), which
 *   it does when the staged INT8 activations of all K columns would not fit
 *   in on-chip memory (large M*K).  Its first 256 KiB hold arrival counters
 *   (one 32-bit counter per row block and chunk of up to 64 tokens, at most
 *   65536 per launch;
 *   calls with more take several launches), the rest the chunks' FP32 sums.
 *   The counters must be zero before the first decode call that uses the
 *   workspace (e.g. a zero-filled allocation); every decode call leaves them
 *   zero, so one workspace serves calls of any projection.  Decode calls
 *   that share a workspace must not run concurrently.
 *   The hand-over between chunks rests on the gfx950 memory system, not on
 *   C++ release/acquire: each workgroup writes its sums with device-scope
 *   stores (sc1), waits until they have completed (vmcnt(0)) before the
 *   barrier that precedes a relaxed device-scope fetch-add of its row
 *   block's counter, and the workgroup that arrives last reads the sums with
 *   device-scope loads.  Device-scope accesses bypass the caches that are
 *   not coherent across the GPU, so a completed store is visible to every
 *   later device-scope load and no cache write-back or invalidation is
 *   issued.
 *   Prefill needs one for a long prompt (M >= 1024) on a projection that
 *   holds INT4 tiles: the temporary INT8 operand of App. E.3 (Prefill), N*K
 *   bytes of INT8 tiles in logical tile order, rounded up to 256, plus
 *   4*N*(K/bK) bytes of scales; its contents need no initialization and are
 *   overwritten by every call that uses it.  A prompt on the decode
 *   kernels (at most 64 rows, or 128 on narrow projections) needs the
 *   decode workspace of the
 *   adaptive split when that plan hands sums over (the larger of the plain
 *   and the transformed plan); the call zeroes its counters itself, so here
 *   too the contents need no initialization. */
size_t aq_workspace_bytes(const aq_packed *W, int M, int phase, int split);

/* Split count that aq_linear_decode uses for `split` = 0: the number of
 * input-column groups each 16-row output group is divided into inside one
 * workgroup (adaptive, chosen from the projection geometry and M). */
int aq_decode_split(const aq_packed *W, int M);

/* Memory-bound phase (Sec. 3.3 "Decode parallelism"; App. E.3 Table 5):
 *   Y[m,n] = sx[m] * sum_j sW[n,j] * P[m,n,j]  (+ bias[n]),
 * P[m,n,j] the INT32 product of the INT8 activation codes and the tile's
 * codes widened to INT8 (eq. 19).  Work is spread over output features and
 * input-column groups: the columns of each 16-row output group are cut into
 * Z workgroup chunks of S splits each, split s of the Z*S covering
 * input-tile columns floor(C*s/(Z*S)) .. floor(C*(s+1)/(Z*S))-1, and the
 * FP32 partials of the splits are summed in increasing s (App. E.3): inside
 * a workgroup through on-chip memory, across chunks by the workgroup that
 * finishes its row block last, all in one kernel launch.  Z = 1 unless
 * aq_workspace_bytes(W, M, 0, split) is non-zero.
 *   qx    device INT8 [M][K] (from aq_quant_act);  sx device FP32 [M]
 *   bias  device FP32 [N] or NULL
 *   Y     device FP32 [M][N] row-major (written, not accumulated)
 *   split 0 = adaptive (aq_decode_split); otherwise S, which must be 16, 8
 *         or 4 (16 waves per workgroup, 1, 2 or 4 row groups; other values
 *         return AQ_ERR_ARG); Z is then the fewest chunks whose
 *         activations fit on chip
 *   ws    device workspace of at least aq_workspace_bytes(W, M, 0, split)
 *         bytes, 16-byte aligned, counters zero (NULL when that is 0), else
 *         AQ_ERR_WORKSPACE
 * Any M >= 1 is accepted (tokens are processed 64 at a time); M == 0 is a
 * no-op. */
aq_status aq_linear_decode(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                           const float *bias, float *Y, int split, void *ws, size_t ws_bytes,
                           void *stream);

/* Decode from FP32 activations: the per-token quantization of
 * aq_quant_act (App. B.3, eq. 5 rounding) followed by aq_linear_decode, in
 * one call.  Y is bit for bit that of aq_quant_act then aq_linear_decode
 * with the same split and bias.  Up to 4 tokens with M*K <= 8192 (so
 * K <= 4096 at M = 2, K <= 8192 at M = 1) run as one kernel: every
 * workgroup quantizes the tokens' rows into on-chip memory as its first
 * weight loads land, which saves the quantizer's launch.  Other calls run
 * aq_quant_act into the workspace, then aq_linear_decode.
 *   X     device FP32 [M][K] row-major, 16-byte aligned
 *   bias, Y, split as aq_linear_decode
 *   ws    device workspace of at least
 *         aq_workspace_bytes(W, M, AQ_PHASE_DECODE_FP32, split) bytes,
 *         16-byte aligned (NULL when that is 0, as for the one-kernel
 *         route), else AQ_ERR_WORKSPACE.  Layout: aq_linear_decode's
 *         workspace first, at least its 256 KiB block of arrival counters
 *         (zero before the call and left zero by it, so one workspace can
 *         serve this call and aq_linear_decode alike), then the INT8 rows
 *         and the FP32 scales, whose contents need no initialization.
 * M == 0 is a no-op. */
aq_status aq_linear_decode_fp32(const aq_packed *W, const float *X, int M, const float *bias, float *Y,
                                int split, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * aq_linear_decode with the workspace taken from a device array inside the
 * library, AQ_DECODE_SCRATCH_BYTES (8 MiB) per GPU, held from the first call
 * on a GPU until the process ends.  The call allocates nothing.  The same
 * kernels, hence the same Y bit for bit, as aq_linear_decode with a
 * workspace.
 *  - A call whose workspace (aq_workspace_bytes(W, M, 0, split)) exceeds
 *    AQ_DECODE_SCRATCH_BYTES returns AQ_ERR_WORKSPACE and launches nothing
 *    (every shape up to 5120 x 17408 fits at M <= 64).
 *  - The first call on a GPU finds the array's address and enqueues on
 *    `stream` a small kernel that zeroes its arrival counters; every call
 *    leaves them zero again.
 *  - All calls on one GPU share the array: calls that overlap in time on
 *    one GPU (other streams, other threads) race and must not be issued.
 * Other arguments and errors as aq_linear_decode. */
#define AQ_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
aq_status aq_linear_decode_noalloc(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                   const float *bias, float *Y, int split, void *stream);

/* Compute-bound phase (Sec. 3.3 "Prefill weight reuse"; App. E.3): the same
 * Y as aq_linear_decode, computed with INT8 matrix-core (MFMA) tiles that
 * reuse each weight tile across many activation rows.  Short prompts
 * (M < 1024) widen the mixed tiles on chip; up to 64 rows (128 on
 * projections whose GEMM grid would not fill half of the compute units)
 * they run on the decode kernels.  Long prompts
 * (M >= 1024, with
 * M*K and N*K below 2^31) first prepare the selected weights as INT8 tiles
 * in logical tile order, once per call, in the workspace (App. E.3
 * Prefill), then run the GEMM over them; a projection without INT4 tiles
 * already stores its W8 buffer in that order and needs no workspace.
 *   ws    device workspace of at least aq_workspace_bytes(W, M, 1, 0) bytes,
 *         16-byte aligned (NULL when that is 0), else AQ_ERR_WORKSPACE
 * Other arguments as aq_linear_decode.  Any M >= 1 is accepted. */
aq_status aq_linear_prefill(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                            const float *bias, float *Y, void *ws, size_t ws_bytes, void *stream);

/* The long-prompt operand preparation of aq_linear_prefill alone (App. E.3
 * Prefill): writes the temporary INT8 operand of a projection with INT4
 * tiles to ws.  It depends on the weights only: a chunked long prompt can
 * prepare it once and run every chunk's GEMM over it, and a caller can
 * prepare the next projection's operand ahead of its activations.
 * A no-op (AQ_OK, nothing launched) when aq_workspace_bytes(W, 1024, 1, 0)
 * is 0: no INT4 tile, or no long route for this geometry.
 *   ws    device workspace of at least aq_workspace_bytes(W, 1024, 1, 0)
 *         bytes, 16-byte aligned, else AQ_ERR_WORKSPACE */
aq_status aq_prefill_prepare(const aq_packed *W, void *ws, size_t ws_bytes, void *stream);

/* aq_linear_prefill over an operand that aq_prefill_prepare has already
 * written to ws for the same W; the caller orders the two (same stream, or
 * an event), and keeps ws unchanged until this call's kernels have run.
 * Prompts that take the short route (M < 1024) do not read ws.  The same
 * kernels as aq_linear_prefill, so the same Y bit for bit.  Arguments and
 * errors as aq_linear_prefill. */
aq_status aq_linear_prefill_prepared(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                     const float *bias, float *Y, const void *ws, size_t ws_bytes,
                                     void *stream);

/* Debug: the INT32 tile products P[m, n, j] of eq. 19 (the parenthesized
 * product, before any scaling), written to P as INT32 [M][N][C] row-major,
 * computed by the decode (phase 0) or prefill (phase 1) kernels themselves,
 * on the same route aq_linear_prefill takes for M rows.
 *   ws    phase 1: workspace as for aq_linear_prefill (phase 0: unused) */
aq_status aq_linear_tile_partials(const aq_packed *W, const int8_t *qx, int M, int phase,
                                  int32_t *P, void *ws, size_t ws_bytes, void *stream);

/* ---- The pages' activation quantizer (App. B.3) ------------------------
 * The entry points above scale activations per token (absmax / 127).  These
 * follow App. B.3 instead: one scale per group of 64 features x b_M rows,
 * b_M = 1 when M == 1 and 16 otherwise, with the endpoint scale of App. B.2
 * eq. 6 at 8 bits, and eq. 19 with one activation scale per 64-feature
 * group (a b_K = 128 tile holds two). */

/* Host only.  Shape of the App. B.3 activation-scale array for M rows of K
 * features: *bM receives b_M (1 when M == 1, otherwise 16), *rows the
 * number of b_M-row groups ceil(M / b_M), *cols the number of 64-feature
 * groups K / 64.  The array that aq_quant_act_grouped writes and the
 * *_grouped linears read is FP32 [rows][cols].  M == 0 gives rows = 0.
 * AQ_ERR_NULL if an output pointer is NULL; AQ_ERR_SHAPE if M < 0, K <= 0
 * or K is not a multiple of 64.  Does not touch the GPU. */
aq_status aq_act_group_shape(int M, int K, int *bM, int *rows, int *cols);

/* Activation quantization with App. B.3 groups: for each group A of b_M rows
 * (rows past M are App. B.3's zero padding) and features 64c .. 64c+63,
 * s = max(max(0, max A) / 127, max(0, -min A) / 128, 1e-12) in FP64 (eq. 6),
 * codes clip(round_half_even(A / s), -128, 127) in FP64 (eq. 5), stored
 * scale FP32(s).
 *   X    device FP32 [M][K], K a multiple of 64
 *   qx   device INT8 [M][K]
 *   sxg  device FP32 [ceil(M/b_M)][K/64] (aq_act_group_shape): group (g, c)
 *        at g*(K/64) + c
 * M == 0 is a no-op. */
aq_status aq_quant_act_grouped(const float *X, int M, int K, int8_t *qx, float *sxg, void *stream);

/* aq_linear_decode with App. B.3 activation groups:
 *   Y[m,n] = sum_c sxg[m / b_M][c] * sW[n, 64c / bK] * P[m,n,c]  (+ bias[n]),
 * P[m,n,c] the INT32 product over the 64 features of group c, summed in the
 * same split order.  sxg as written by aq_quant_act_grouped for the same M.
 * split, ws and errors as aq_linear_decode (the same workspace rule).  The
 * host metadata image (aq_packed.meta_host) is not used on this route. */
aq_status aq_linear_decode_grouped(const aq_packed *W, const int8_t *qx, const float *sxg, int M,
                                   const float *bias, float *Y, int split, void *ws, size_t ws_bytes,
                                   void *stream);

/* The same product for any prompt length.  Long prompts (the long route of
 * aq_linear_prefill, at b_K = 128) run the long-prompt GEMM: the temporary
 * INT8 operand (App. E.3 Prefill), then the 256 x 128 MFMA GEMM with the two
 * 64-feature halves of every 128-column tile kept as separate INT32
 * products, each rescaled by its activation-group scale times the row's
 * weight scale (eq. 19 per group).  Shorter prompts run the decode kernels
 * (up to 64 tokens per workgroup, token chunks one after another), exactly
 * as aq_linear_decode_grouped with split 0.
 *   ws    at least aq_workspace_bytes(W, M, AQ_PHASE_PREFILL_GROUPED, 0)
 *         bytes, 16-byte aligned (NULL when that is 0): the temporary operand
 *         on the long route, else the decode workspace (its counters zero, as
 *         for aq_linear_decode), else AQ_ERR_WORKSPACE */
aq_status aq_linear_prefill_grouped(const aq_packed *W, const int8_t *qx, const float *sxg, int M,
                                    const float *bias, float *Y, void *ws, size_t ws_bytes,
                                    void *stream);

/* Debug: the INT32 group products P[m, n, c] of the grouped eq. 19, written
 * as INT32 [M][N][K/64] row-major by the kernels aq_linear_prefill_grouped
 * takes for M rows (the long-prompt GEMM, or the grouped decode kernels).
 *   ws    on the long route, a workspace as for aq_linear_prefill_grouped
 *         (otherwise unused) */
aq_status aq_linear_tile_partials_grouped(const aq_packed *W, const int8_t *qx, int M, int32_t *P, void *ws,
                                          size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Tile-aligned orthogonal transforms (App. B.1, eq. 4).
 *
 * Each 64-block transform is Phi_s, s in -1 .. 6: Phi_-1 = I, Phi_0 = H_64
 * (Sylvester order, entries +-1/8), and for s >= 1 the signed permutation
 * Phi_s = D_L,s P_s H_64 D_R,s with (P_s v)_i = v[perm[s-1][i]] and the
 * diagonals dl[s-1], dr[s-1] of +-1.  The pages fix the form, not P_s and
 * the signs, so the caller supplies them.  The activation transform
 * V = diag(Phi_{v_c}) acts on 64-feature blocks c; the output transform
 * U = diag(Phi_{u_r}^T) on 64-row output tile rows r.  The transformed layer
 * is W~ = U W V, X~ = X V, and Y = Y~ U recovers the output.
 *
 * FP32 evaluation order (X~ and W~ feed quantizers, so it is fixed): signs
 * and the permutation are exact; H_64 is six in-place butterfly stages,
 * h = 1, 2, 4, .., 32, (a_i, a_i+h) -> (a_i + a_i+h, a_i - a_i+h) for each
 * i with bit h clear, then the exact factor 1/8.
 *
 * Seeds are device INT8 arrays; a seed outside -1 .. 6 turns the block(s) it
 * governs into NaN.  The tables are read on the host at the call and
 * checked: every perm row a permutation of 0 .. 63, every sign +-1, else
 * AQ_ERR_ARG (NULL tables: AQ_ERR_NULL).  They are copied into the launch,
 * so the host memory may be reused as soon as the call returns.
 * ------------------------------------------------------------------------- */
#define AQ_TRANSFORM_SEEDS 6
typedef struct aq_transform_tables {
  uint8_t perm[AQ_TRANSFORM_SEEDS][64];
  int8_t dl[AQ_TRANSFORM_SEEDS][64];
  int8_t dr[AQ_TRANSFORM_SEEDS][64];
} aq_transform_tables;

/* X~ = X V: every 64-feature block c of every row x becomes Phi_{v_c}^T x.
 *   X, Xt    device FP32 [M][K], K a multiple of 64; Xt == X is allowed
 *   vseeds   device INT8 [K/64]
 * M == 0 is a no-op. */
aq_status aq_transform_rows(const float *X, int M, int K, const int8_t *vseeds,
                            const aq_transform_tables *tables_host, float *Xt, void *stream);

/* Y = Y~ U (+ bias): every 64-feature block r of every output row y~
 * becomes Phi_{u_r} y~ (eq. 4), then bias[n] is added.  The bias belongs to
 * the untransformed output, so a transformed layer passes it here and not
 * to the linear call.
 *   Yt, Y    device FP32 [M][N], N a multiple of 64; Y == Yt is allowed
 *   useeds   device INT8 [N/64]
 *   bias     device FP32 [N] or NULL
 * M == 0 is a no-op. */
aq_status aq_transform_out(const float *Yt, int M, int N, const int8_t *useeds,
                           const aq_transform_tables *tables_host, const float *bias, float *Y,
                           void *stream);

/* The transformed layer's prefill linear (App. B.1 eq. 4 around App. E.3
 * eq. 19): Y = Y~ U + bias, Y~ the
 * aq_linear_prefill product of the transformed operands (W~ packed, qx / sx
 * from aq_quant_act_transformed).  Every route of aq_linear_prefill (the
 * short-prompt GEMM, and for long prompts the GEMM kernel the plain call
 * takes) applies U in its epilogue, where each wave holds the 64 outputs of
 * a tile row per token, before the token scale and the bias.  Within FP32
 * rounding of aq_linear_prefill followed by aq_transform_out.
 *   useeds   device INT8 [N/64];  tables_host as for the transforms
 * Other arguments, workspace and errors as aq_linear_prefill. */
aq_status aq_linear_prefill_transformed(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                        const float *bias, const int8_t *useeds,
                                        const aq_transform_tables *tables_host, float *Y, void *ws,
                                        size_t ws_bytes, void *stream);

/* The transformed layer's decode linear (App. B.1 eq. 4 in the epilogue of
 * App. E.3 eq. 19): Y = (Y~ U) + bias, Y~ the aq_linear_decode product of
 * the transformed operands.  After the ordered split sum and the token
 * scale, the workgroup that holds the last part of a 64-row tile row
 * applies Phi_{u_r} to its 64 outputs per token, then adds the bias: bit for
 * bit aq_linear_decode (bias NULL) with the same split followed by
 * aq_transform_out (bias), in one launch.  When the decode plan spreads a
 * tile row over several workgroups (row groups in different workgroups, or
 * column chunks), their sums meet in the workspace as for chunked K, with
 * one arrival counter per tile row and token chunk.  split = 0 takes the
 * adaptive split of aq_linear_decode, except that it keeps a tile row's four
 * row groups in one workgroup (split 4) where each wave's share of the
 * row then still fits one batch of weight loads.
 *   useeds   device INT8 [N/64];  tables_host as for the transforms
 *   ws       device workspace of at least
 *            aq_workspace_bytes(W, M, AQ_PHASE_DECODE_TRANSFORMED, split)
 *            bytes, 16-byte aligned, counters zero (NULL when that is 0),
 *            else AQ_ERR_WORKSPACE; decode and transformed decode calls may
 *            share one workspace (neither leaves a counter set)
 * Other arguments and errors as aq_linear_decode.  Multi-chunk calls (more
 * than 64 tokens) load the weights non-temporally in every chunk. */
aq_status aq_linear_decode_transformed(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                       const float *bias, const int8_t *useeds,
                                       const aq_transform_tables *tables_host, float *Y, int split,
                                       void *ws, size_t ws_bytes, void *stream);

/* aq_quant_act of X~ = X V in one pass: the same codes and scales as
 * aq_transform_rows followed by aq_quant_act, bit for bit, with the
 * transformed rows kept on chip (read X once, write the codes once).
 *   X        device FP32 [M][K], K a multiple of 64 and at most 40768 (one
 *            transformed row is staged in 160 KiB of LDS; longer rows take
 *            the two calls)
 *   vseeds   device INT8 [K/64]
 *   qx, sx   as aq_quant_act
 * A seed outside -1 .. 6 makes that row's scale NaN.  M == 0 is a no-op. */
aq_status aq_quant_act_transformed(const float *X, int M, int K, const int8_t *vseeds,
                                   const aq_transform_tables *tables_host, int8_t *qx, float *sx,
                                   void *stream);

/* W~ = U W V: first each row's 64-feature blocks by Phi_{v_c}^T (as
 * aq_transform_rows), then the 64 rows of each output tile row r, column by
 * column, by U_r = Phi_{u_r}^T.
 *   W, Wt    device FP32 [N][K], N and K multiples of 64; Wt must not
 *            overlap W
 *   useeds   device INT8 [N/64];  vseeds device INT8 [K/64] */
aq_status aq_transform_weights(const float *W, int N, int K, const int8_t *useeds,
                               const int8_t *vseeds, const aq_transform_tables *tables_host,
                               float *Wt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQ_H */
