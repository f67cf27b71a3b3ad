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
hipError_t launch_quant_act_grouped(const float *X, int M, int K, int8_t *qx, float *sxg,
                                    hipStream_t stream);
hipError_t launch_prefill(const PackedView &w, const int8_t *qx, const float *sx, int M,
                          const float *bias, float *Y, int32_t *P, hipStream_t stream);

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

// Persistent 256 x 256-tile variant of the long-prefill GEMM (b_K = 128,
// N >= 6144, at least one tile per compute unit, M*N < 2^29); same operands;
// P != nullptr writes INT32 products instead of Y.
int compute_units();
bool prefill_big_fits(int N, int K, int bK, int M);
hipError_t launch_prefill_big(const int8_t *E, const float *Es, int N, int K, const int8_t *qx,
                              const float *sx, int M, const float *bias, float *Y, int32_t *P,
                              hipStream_t stream);

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
inline size_t prefill_workspace_bytes(const PackedView &w, int M) {
  return prefill_long(w, M) && w.T4 > 0 ? expand_bytes(w) : 0;
}

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
  size_t lds, cnt_bytes, ws_bytes;
};
// split = 0: adaptive; otherwise S, one of the supported values.
DecodePlan plan_decode(const PackedView &w, int M, int split);
// false when a chunked plan has more row blocks than arrival counters
bool decode_plan_ok(const DecodePlan &p, const PackedView &w);
int decode_split(const PackedView &w, int M);
bool decode_split_supported(const PackedView &w, int M, int S);
size_t decode_workspace_bytes(const PackedView &w, int M, int split);

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

}  // namespace aq
