// Internal interface between the host ABI layer (aq_api.cpp) and the HIP
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/aq.h"

namespace aq {

// Geometry the GPU kernels are built for.
constexpr int kTileRows = 64;  // b_N

// Read-only view of a packed projection plus derived geometry.
struct PackedView {
  int N, K, bK, R, C, T4, T8;
  const uint8_t *labels;
  const int32_t *off4, *off8;
  const uint8_t *w4;
  const int8_t *w8;
  const float *s4, *s8;
  const uint32_t *meta;  // host metadata image, or nullptr
};

inline PackedView view_of(const aq_packed &p) {
  PackedView v;
  v.N = p.N; v.K = p.K; v.bK = p.bK;
  v.R = p.N / kTileRows; v.C = p.K / p.bK;
  v.T4 = p.T4; v.T8 = p.T8;
  v.labels = p.labels; v.off4 = p.row_off4; v.off8 = p.row_off8;
  v.w4 = p.w4; v.w8 = p.w8; v.s4 = p.s4; v.s8 = p.s8;
  v.meta = p.meta_host;
  return v;
}

// Launchers.  Arguments are already validated; each returns the launch
// status reported by hipGetLastError().
// mse: the fitted scale of App. B.2 eq. 7 instead of the absmax scale
hipError_t launch_pack(const float *W, const aq_packed &out, hipStream_t stream, bool mse = false);
hipError_t launch_quant_act(const float *X, int M, int K, int8_t *qx, float *sx,
                            hipStream_t stream);
// Decode: one launch; the input-column splits of each output row group are
// reduced in increasing order, through LDS inside a workgroup and, when the
// plan cuts the columns into Z > 1 workgroup chunks, through the workspace
// (ws, decode_workspace_bytes bytes, counters zero on entry and on exit).
// split 0 = adaptive.  P != nullptr selects the debug mode that writes
// INT32 tile products instead (Y and ws unused).
// grouped: sx holds the App. B.3 activation-group scales ([ceil(M/b_M)][K/64],
// b_M = 1 for M = 1, else 16) and P, when given, is [M][N][K/64].
hipError_t launch_decode(const PackedView &w, const int8_t *qx, const float *sx, int M,
                         const float *bias, float *Y, int split, void *ws, int32_t *P,
                         hipStream_t stream, bool grouped = false);
// App. B.3 activation groups: 64 features x b_M rows, b_M = 1 for a single
// token and 16 otherwise.  The one place the rule lives on the host side;
// the grouped quantizer's launch, the grouped decode launch and
// aq_act_group_shape take it from here.
constexpr int kActGroupK = 64;
inline int act_group_rows(int M) { return M == 1 ? 1 : 16; }
hipError_t launch_quant_act_grouped(const float *X, int M, int K, int8_t *qx, float *sxg,
                                    hipStream_t stream);
// Short prompts: the 32 x 32 MFMA GEMM over the packed tiles; useeds and
// tables (both or neither) apply the output transform in its epilogue, as
// for launch_prefill_dense.
hipError_t launch_prefill(const PackedView &w, const int8_t *qx, const float *sx, int M,
                          const float *bias, float *Y, int32_t *P, hipStream_t stream,
                          const int8_t *useeds = nullptr, const aq_transform_tables *tables = nullptr);

// Long-prefill GEMM over INT8 tiles in logical tile order: E holds tile
// (r, j) at (r*C + j) * 64*bK bytes (b_K/16 panels of [64][16]) and Es its
// 64 FP32 row scales at (r*C + j) * 64.  P != nullptr writes INT32 products.
// useeds (device, R seeds) and tables, when given, apply the output
// transform of App. B.1 (Y = Y~ U) in the epilogue, before the token scale
// and the bias.
hipError_t launch_prefill_dense(const int8_t *E, const float *Es, int N, int K, int bK,
                                const int8_t *qx, const float *sx, int M, const float *bias,
                                float *Y, int32_t *P, hipStream_t stream,
                                const int8_t *useeds = nullptr,
                                const aq_transform_tables *tables = nullptr);

// The long-prefill GEMM with the pages' activation groups (App. B.3; b_K =
// 128, M >= 2): sxg [ceil(M/16)][K/64]; P != nullptr writes the INT32
// group products [M][N][K/64] instead of Y.
hipError_t launch_prefill_dense_grouped(const int8_t *E, const float *Es, int N, int K, const int8_t *qx,
                                        const float *sxg, int M, const float *bias, float *Y, int32_t *P,
                                        hipStream_t stream);

// Persistent 256 x 256-tile variant of the long-prefill GEMM (b_K = 128,
// N >= 6144, tiles for at least half of the compute units, M*N < 2^29); same operands;
// P != nullptr writes INT32 products instead of Y; useeds and tables as for
// launch_prefill_dense.
int compute_units();
bool prefill_big_fits(int N, int K, int bK, int M);
hipError_t launch_prefill_big(const int8_t *E, const float *Es, int N, int K, const int8_t *qx,
                              const float *sx, int M, const float *bias, float *Y, int32_t *P,
                              hipStream_t stream, const int8_t *useeds = nullptr,
                              const aq_transform_tables *tables = nullptr);

// Temporary INT8 operand of long prefill: bytes of the buffer (INT8 tiles in
// logical order, then FP32 scales), and the launch that fills it from the
// packed model; *E / *Es receive the two parts inside ws.
size_t expand_bytes(const PackedView &w);
hipError_t launch_expand(const PackedView &w, void *ws, hipStream_t stream, const int8_t **E,
                         const float **Es);
// Where launch_expand puts the two parts inside ws (no launch).
void expand_layout(const PackedView &w, const void *ws, const int8_t **E, const float **Es);

// Prefill routing: prompts of at least kLongPrefillM rows run the GEMM over
// INT8 tiles in logical order (the packed W8 buffer itself when the map has
// no INT4 tile, else the temporary buffer); shorter ones prepare the mixed
// tiles on chip.  The dense GEMM addresses operands with 32-bit offsets.
constexpr int kLongPrefillM = 1024;
inline bool prefill_long(const PackedView &w, int M) {
  return M >= kLongPrefillM && (long long)M * w.K < (1LL << 31) &&
         (long long)w.N * w.K < (1LL << 31);
}
// Prompts of at most kPrefillDecodeMaxM rows run on the decode kernels: the
// short-prompt GEMM has one 128-token block row there, too few blocks to
// fill the chip.  A decode plan that hands sums over gets its workspace from
// the prefill call, whose arrival counters the call zeroes first (prefill
// workspaces need no initialization).  xform: the plan of the transformed
// decode.
constexpr int kPrefillDecodeMaxM = 64;
// ... and up to kPrefillDecodeNarrowM rows on projections whose GEMM grid
// (one block per 128 tokens x 2 tile rows) would not reach half of the CUs
constexpr int kPrefillDecodeNarrowM = 128;
bool prefill_on_decode(const PackedView &w, int M, bool xform = false);
// Workspace of a prefill call (aq_linear_prefill, its transformed variant):
// the temporary operand of long prompts, or the decode kernels' workspace of
// short prompts on them (the larger of the plain and transformed plans).
size_t prefill_call_workspace_bytes(const PackedView &w, int M);
// Zeroes the arrival counters at the head of a decode workspace (a fill
// kernel, so that it can be captured into a graph).
hipError_t launch_zero_counters(void *ws, hipStream_t stream);
// Grouped activations (App. B.3) take the long-prompt GEMM for long prompts
// at b_K = 128; otherwise the decode kernels.
inline bool prefill_grouped_long(const PackedView &w, int M) { return w.bK == 128 && prefill_long(w, M); }
inline size_t prefill_workspace_bytes(const PackedView &w, int M) {
  return prefill_long(w, M) && w.T4 > 0 ? expand_bytes(w) : 0;
}

// Decode geometry shared by the kernels (aq_decode.hip) and the host
// planner (aq_plan.cpp).
constexpr int kLdsBudget = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kValuMaxM = 1;            // largest M on the vector-ALU path
constexpr int kPrivMaxM = 4;            // largest M with per-wave activation slices of 8 tiles
constexpr int kPrivDepth = 8;           // tiles per batch with per-wave activation slices
// Per-wave slices of 4 tiles for up to 16 tokens, where every wave's share
// of the columns is one batch (b_K = 128)
constexpr int kPriv16MaxM = 16;
constexpr int kPriv16Depth = 4;
constexpr int kSharedDepth1 = 8;        // tiles per batch, shared staging, one token group
constexpr int kSharedDepthN = 6;        // tiles per batch, shared staging, 2 token groups
constexpr int kSharedDepthW = 4;        // tiles per batch, shared staging, 3-4 token groups
constexpr int kDecodeCounters = 65536;  // arrival counters at the head of a decode workspace
constexpr int kInlineWords = 896;       // metadata words that may travel in the kernel arguments
constexpr int kInlineWordsXf = 768;     // the same with the output-transform tables beside them
constexpr int kMetaStride = 6;          // words per tile row in the host metadata image
enum { kValu = 0, kMfma = 1 };
// Where the MFMA/VALU activation operands come from: a per-wave LDS slice
// of the batch, the workgroup's LDS copy of its tokens' chunk columns, or
// that copy quantized by the workgroup itself from the FP32 activations.
enum { kXPriv = 0, kXShared = 1, kXFused = 2 };
// The fused route quantizes at most kFusedMaxM tokens, whose FP32 rows are
// loaded once, kFusedUnits float4 per thread of the 16-wave workgroup
// (M * K <= 4 * 1024 * kFusedUnits).  Every workgroup quantizes all of them:
// measured on the Llama-3.2-3B-shaped projections, the route beats the
// separate quantizer launch by 0.7-1.0 us per call at M = 1 and 0.3-0.5 us
// at M = 2, K = 3072, and loses 0.8 us beyond 8192 elements (K = 8192,
// M = 2).
constexpr int kFusedMaxM = 4;
constexpr int kFusedUnits = 2;

// Launch plan of one decode call: products on the vector ALU or MFMA, where
// the activation operands live, token groups of 16 per workgroup, waves,
// row groups RG and splits S = waves / RG per workgroup, input-column
// chunks Z (one workgroup each), token chunks, dynamic LDS bytes, the LDS
// row stride of staged activations, and the workspace (arrival counters,
// then FP32 chunk sums) that Z > 1 needs.
// A chunked call's workspace starts with a fixed 256 KiB of arrival
// counters (one per row block and token chunk of a launch); token chunks
// beyond that take further launches of ylaunch chunks each.
struct DecodePlan {
  int mode, xmode, MG, waves, RG, S, Z, mchunks, ylaunch, xstride;
  int depth;  // tiles per batch of the per-wave slices (kPrivDepth or kPriv16Depth)
  size_t lds, cnt_bytes, ws_bytes;
};
// split = 0: adaptive; otherwise S, one of the supported values.  xform:
// the call applies the output transform in its epilogue, which needs the
// whole 64-row tile row in one workgroup; when the plan spreads a tile row
// over several workgroups (RG < 4 or Z > 1), their sums meet in the
// workspace (counters per tile row and token chunk, then the sums) and the
// last of them finishes the tile row.
DecodePlan plan_decode(const PackedView &w, int M, int split, bool xform = false);
// false when a plan that hands sums over needs more arrival counters than
// the workspace holds
bool decode_plan_ok(const DecodePlan &p, const PackedView &w, bool xform = false);
int decode_split(const PackedView &w, int M);
bool decode_split_supported(const PackedView &w, int M, int S);
size_t decode_workspace_bytes(const PackedView &w, int M, int split, bool xform = false);
// Decode from FP32 activations.  fused_ok: the call fits the one-kernel
// route (at most kFusedMaxM tokens, rows within the per-thread loads and
// LDS, no column chunks), whose plan is plan_decode_fused: the per-token
// plan's row groups and splits, the tokens' quantized rows shared in LDS.
// Otherwise launch_decode_fp32 quantizes into the workspace and runs the
// decode linear: the decode workspace first, at least the whole block of
// arrival counters (fp32_head_bytes, so that a workspace shared with other
// decode calls keeps zero counters), then the INT8 rows and the scales;
// fp32_workspace_bytes covers both routes.
bool fused_ok(const PackedView &w, int M, int split);
DecodePlan plan_decode_fused(const PackedView &w, int M, int split);
size_t fp32_head_bytes(const PackedView &w, int M, int split);
size_t fp32_workspace_bytes(const PackedView &w, int M, int split);
hipError_t launch_decode_fp32(const PackedView &w, const float *X, int M, const float *bias, float *Y,
                              int split, void *ws, hipStream_t stream);
// The allocation-free decode's device scratch (AQ_DECODE_SCRATCH_BYTES):
// its address on the current device, found once per device with
// hipGetSymbolAddress; the first call on a device also enqueues, on
// `stream`, a fill kernel that zeroes the arrival counters at its head.
constexpr size_t kDecodeScratchBytes = AQ_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(hipStream_t stream, void **out);

// Block transforms of App. B.1 (kind: rows = X V, out = Y~ U, weights =
// U W V); seeds2 is the per-tile-row seed array of the weight transform.
using TransformTables = aq_transform_tables;
constexpr int kTransformSeeds = AQ_TRANSFORM_SEEDS;
enum { kTransformRows = 0, kTransformOut = 1, kTransformWeights = 2 };
hipError_t launch_transform(int kind, const float *src, float *dst, int rows, int cols,
                            const int8_t *seeds, const int8_t *seeds2, const float *bias,
                            const TransformTables &t, hipStream_t stream);
// X V and the per-token quantizer in one pass; the transformed row is staged
// in LDS (160 KiB less the tables and the reduction slots), so K is bounded
// by kQuantTransformMaxK.
constexpr int kQuantTransformMaxK = 40768;
hipError_t launch_quant_act_transformed(const float *X, int M, int K, const int8_t *seeds,
                                        const TransformTables &t, int8_t *qx, float *sx,
                                        hipStream_t stream);
// Decode with the output transform in the epilogue: the same sums as
// launch_decode, scaled by sx, then Y~ U per tile row (useeds: device, R
// seeds), then the bias; bit for bit launch_decode without the bias
// followed by launch_transform(kTransformOut) with it.  ws as
// decode_workspace_bytes(w, M, split, true).
hipError_t launch_decode_transformed(const PackedView &w, const int8_t *qx, const float *sx, int M,
                                     const float *bias, float *Y, int split, void *ws,
                                     const int8_t *useeds, const TransformTables &t,
                                     hipStream_t stream);

}  // namespace aq
