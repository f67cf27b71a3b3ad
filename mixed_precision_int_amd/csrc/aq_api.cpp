// Host side of the C ABI declared in include/aq.h: argument validation,
// planning, metadata upload and kernel dispatch.  Everything is checked
// before any HIP call is made, so invalid calls never touch the GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/aq.h"
#include "aq_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int bit_of(const uint8_t *labels, int t) { return (labels[t >> 3] >> (t & 7)) & 1; }

// Geometry accepted by the GPU kernels.
aq_status check_gpu_geometry(int N, int K, int bN, int bK) {
  if (bN != aq::kTileRows || (bK != 64 && bK != 128)) return AQ_ERR_TILE;
  if (N <= 0 || K <= 0 || N % bN || K % bK) return AQ_ERR_SHAPE;
  // int32 tile counts and K-offsets inside kernels
  if ((long long)(N / bN) * (K / bK) > (1LL << 30)) return AQ_ERR_SHAPE;
  return AQ_OK;
}

aq_status check_packed(const aq_packed *W) {
  if (!W) return AQ_ERR_NULL;
  aq_status st = check_gpu_geometry(W->N, W->K, W->bN, W->bK);
  if (st != AQ_OK) return st;
  const long long T = (long long)(W->N / W->bN) * (W->K / W->bK);
  if (W->T4 < 0 || W->T8 < 0 || (long long)W->T4 + W->T8 != T) return AQ_ERR_MAP;
  if (!W->labels || !W->row_off4 || !W->row_off8) return AQ_ERR_NULL;
  if (!aligned4(W->labels)) return AQ_ERR_ALIGN;
  if (W->T4 > 0 && (!W->w4 || !W->s4)) return AQ_ERR_NULL;
  if (W->T8 > 0 && (!W->w8 || !W->s8)) return AQ_ERR_NULL;
  if (!aligned4(W->row_off4) || !aligned4(W->row_off8)) return AQ_ERR_ALIGN;
  if (W->meta_host && !aligned4(W->meta_host)) return AQ_ERR_ALIGN;
  if (W->T4 > 0 && (!aligned16(W->w4) || !aligned16(W->s4))) return AQ_ERR_ALIGN;
  if (W->T8 > 0 && (!aligned16(W->w8) || !aligned16(W->s8))) return AQ_ERR_ALIGN;
  return AQ_OK;
}

aq_status check_linear_io(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                          const float *bias, const void *out) {
  if (M < 0) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!qx || !sx || !out) return AQ_ERR_NULL;
  if (!aligned16(qx) || !aligned16(out) || !aligned4(sx)) return AQ_ERR_ALIGN;
  if (bias && !aligned16(bias)) return AQ_ERR_ALIGN;
  // 64-bit products are used for every offset; keep each dimension sane.
  if ((long long)M * W->K > (1LL << 40) || (long long)M * W->N > (1LL << 40)) return AQ_ERR_SHAPE;
  return AQ_OK;
}

aq_status check_workspace(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return AQ_OK;
  if (!ws || ws_bytes < need) return AQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return AQ_ERR_ALIGN;
  return AQ_OK;
}

// Prefill dispatch (Y, or INT32 products into P when P != nullptr).
// prepared: ws already holds the temporary INT8 operand (aq_prefill_prepare).
hipError_t run_prefill(const aq::PackedView &v, const int8_t *qx, const float *sx, int M,
                       const float *bias, float *Y, int32_t *P, void *ws, hipStream_t s,
                       bool prepared = false) {
  if (!aq::prefill_long(v, M)) {
    if (aq::prefill_on_decode(v, M)) {
      // the products need no hand-over; a prepared workspace holds the
      // operand and is not the decode kernels' to use
      const size_t need = P ? 0 : aq::decode_workspace_bytes(v, M, 0);
      if (need == 0) return aq::launch_decode(v, qx, sx, M, bias, Y, 0, nullptr, P, s);
      if (!prepared) {
        const hipError_t e = aq::launch_zero_counters(ws, s);
        if (e != hipSuccess) return e;
        return aq::launch_decode(v, qx, sx, M, bias, Y, 0, ws, nullptr, s);
      }
    }
    return aq::launch_prefill(v, qx, sx, M, bias, Y, P, s);
  }
  const int8_t *E = v.w8;
  const float *Es = v.s8;
  if (v.T4 > 0 && prepared) {
    aq::expand_layout(v, ws, &E, &Es);
  } else if (v.T4 > 0) {
    const hipError_t e = aq::launch_expand(v, ws, s, &E, &Es);
    if (e != hipSuccess) return e;
  }
  if (aq::prefill_big_fits(v.N, v.K, v.bK, M))
    return aq::launch_prefill_big(E, Es, v.N, v.K, qx, sx, M, bias, Y, P, s);
  return aq::launch_prefill_dense(E, Es, v.N, v.K, v.bK, qx, sx, M, bias, Y, P, s);
}

// Long grouped prefill: the temporary operand as for run_prefill, then the
// 256 x 128 GEMM with App. B.3 activation groups (Y, or the INT32 group
// products into P).
hipError_t run_prefill_grouped(const aq::PackedView &v, const int8_t *qx, const float *sxg, int M,
                               const float *bias, float *Y, int32_t *P, void *ws, hipStream_t s) {
  const int8_t *E = v.w8;
  const float *Es = v.s8;
  if (v.T4 > 0) {
    const hipError_t e = aq::launch_expand(v, ws, s, &E, &Es);
    if (e != hipSuccess) return e;
  }
  return aq::launch_prefill_dense_grouped(E, Es, v.N, v.K, qx, sxg, M, bias, Y, P, s);
}

}  // namespace

extern "C" {

int aq_abi_version(void) { return AQ_ABI_VERSION; }

const char *aq_status_string(aq_status s) {
  switch (s) {
    case AQ_OK: return "ok";
    case AQ_ERR_NULL: return "a required pointer is NULL";
    case AQ_ERR_SHAPE: return "shape not compatible with the tile geometry";
    case AQ_ERR_TILE: return "tile size not supported (GPU: b_N = 64, b_K in {64, 128})";
    case AQ_ERR_MAP: return "labels disagree with T4/T8 or a map entry is not 4 or 8";
    case AQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case AQ_ERR_WORKSPACE: return "workspace missing or too small";
    case AQ_ERR_HIP: return "HIP runtime error at launch";
    case AQ_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

aq_status aq_labels_from_map(const uint8_t *zmap, int R, int C, uint8_t *labels) {
  if (!zmap || !labels) return AQ_ERR_NULL;
  if (R <= 0 || C <= 0) return AQ_ERR_SHAPE;
  const long long T = (long long)R * C;
  for (long long b = 0; b < (T + 7) / 8; ++b) labels[b] = 0;
  for (long long t = 0; t < T; ++t) {
    if (zmap[t] == 4) labels[t >> 3] |= (uint8_t)(1u << (t & 7));
    else if (zmap[t] != 8) return AQ_ERR_MAP;
  }
  return AQ_OK;
}

aq_status aq_plan_pack(int N, int K, int bN, int bK, const uint8_t *labels, aq_plan *out) {
  if (!labels || !out) return AQ_ERR_NULL;
  if (bN < 1 || bK < 32 || bK % 32) return AQ_ERR_TILE;
  if (N <= 0 || K <= 0 || N % bN || K % bK) return AQ_ERR_SHAPE;
  const long long R = N / bN, C = K / bK, T = R * C;
  if (T > (1LL << 30)) return AQ_ERR_SHAPE;
  long long T4 = 0;
  for (long long t = 0; t < T; ++t) T4 += bit_of(labels, (int)t);
  aq_plan p;
  p.N = N; p.K = K; p.bN = bN; p.bK = bK;
  p.R = (int32_t)R; p.C = (int32_t)C;
  p.T4 = (int32_t)T4; p.T8 = (int32_t)(T - T4);
  const size_t B = (size_t)bN * bK;
  p.labels_bytes = (size_t)((T + 7) / 8);
  p.labels_alloc = 4 * (size_t)((T + 31) / 32);
  p.offs_bytes = 4 * (size_t)(R + 1);
  p.w4_bytes = B / 2 * (size_t)p.T4;
  p.w8_bytes = B * (size_t)p.T8;
  p.s4_bytes = 4 * (size_t)bN * p.T4;
  p.s8_bytes = 4 * (size_t)bN * p.T8;
  p.meta_bytes = C <= 128 ? 24 * (size_t)R : 0;
  *out = p;
  return AQ_OK;
}

namespace {
aq_status pack_impl(const float *W, const uint8_t *labels_host, aq_packed *out, void *stream,
                    bool mse);
}  // namespace

aq_status aq_pack_weights(const float *W, const uint8_t *labels_host, aq_packed *out,
                          void *stream) {
  return pack_impl(W, labels_host, out, stream, false);
}

aq_status aq_pack_weights_mse(const float *W, const uint8_t *labels_host, aq_packed *out,
                              void *stream) {
  return pack_impl(W, labels_host, out, stream, true);
}

}  // extern "C"

namespace {
aq_status pack_impl(const float *W, const uint8_t *labels_host, aq_packed *out, void *stream,
                    bool mse) {
  if (!W || !labels_host || !out) return AQ_ERR_NULL;
  aq_status st = check_packed(out);
  if (st != AQ_OK) return st;
  if (!aligned16(W)) return AQ_ERR_ALIGN;
  aq_plan plan;
  st = aq_plan_pack(out->N, out->K, out->bN, out->bK, labels_host, &plan);
  if (st != AQ_OK) return st;
  if (plan.T4 != out->T4 || plan.T8 != out->T8) return AQ_ERR_MAP;

  // Row offsets (App. E.2): two INT32 arrays of length R+1; labels padded
  // with zero bytes to whole 32-bit words.
  std::vector<int32_t> offs;
  std::vector<uint8_t> lab;
  try {
    offs.resize(2 * (size_t)(plan.R + 1));
    lab.assign(plan.labels_alloc, 0);
  } catch (const std::bad_alloc &) {
    return AQ_ERR_ARG;
  }
  for (size_t b = 0; b < plan.labels_bytes; ++b) lab[b] = labels_host[b];
  const long long T = (long long)plan.R * plan.C;
  if (T % 8) lab[plan.labels_bytes - 1] &= (uint8_t)((1u << (T % 8)) - 1u);  // unused bits zero
  int32_t *o4 = offs.data(), *o8 = offs.data() + plan.R + 1;
  o4[0] = o8[0] = 0;
  for (int r = 0; r < plan.R; ++r) {
    int c4 = 0;
    for (int j = 0; j < plan.C; ++j) c4 += bit_of(labels_host, r * plan.C + j);
    o4[r + 1] = o4[r] + c4;
    o8[r + 1] = o8[r] + (plan.C - c4);
  }
  if (out->meta_host && plan.meta_bytes) {
    // host image, one 6-word record per tile row: row_off4[r], row_off8[r],
    // then the labels of the row's C <= 128 tiles as 128 bits, LSB first
    uint32_t *m = out->meta_host;
    for (int r = 0; r < plan.R; ++r) {
      uint32_t *rec = m + 6 * (size_t)r;
      rec[0] = (uint32_t)o4[r];
      rec[1] = (uint32_t)o8[r];
      rec[2] = rec[3] = rec[4] = rec[5] = 0u;
      for (int j = 0; j < plan.C; ++j)
        rec[2 + (j >> 5)] |= (uint32_t)bit_of(labels_host, r * plan.C + j) << (j & 31);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(out->labels, lab.data(), plan.labels_alloc, hipMemcpyHostToDevice, s) !=
          hipSuccess ||
      hipMemcpyAsync(out->row_off4, o4, plan.offs_bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(out->row_off8, o8, plan.offs_bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)  // host buffers are released on return
    return AQ_ERR_HIP;
  return aq::launch_pack(W, *out, s, mse) == hipSuccess ? AQ_OK : AQ_ERR_HIP;
}
}  // namespace

extern "C" {

aq_status aq_quant_act(const float *X, int M, int K, int8_t *qx, float *sx, void *stream) {
  if (M < 0 || K <= 0 || K % 64) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!X || !qx || !sx) return AQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(qx) || !aligned4(sx)) return AQ_ERR_ALIGN;
  if ((long long)M * K > (1LL << 40) || M > (1 << 30)) return AQ_ERR_SHAPE;
  return aq::launch_quant_act(X, M, K, qx, sx, static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_act_group_shape(int M, int K, int *bM, int *rows, int *cols) {
  if (!bM || !rows || !cols) return AQ_ERR_NULL;
  if (M < 0 || K <= 0 || K % aq::kActGroupK) return AQ_ERR_SHAPE;
  const int b = aq::act_group_rows(M);
  *bM = b;
  *rows = M / b + (M % b != 0);
  *cols = K / aq::kActGroupK;
  return AQ_OK;
}

aq_status aq_quant_act_grouped(const float *X, int M, int K, int8_t *qx, float *sxg, void *stream) {
  if (M < 0 || K <= 0 || K % 64) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!X || !qx || !sxg) return AQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(qx) || !aligned4(sxg)) return AQ_ERR_ALIGN;
  if ((long long)M * K > (1LL << 40) || (M + 15) / 16 > 65535) return AQ_ERR_SHAPE;
  return aq::launch_quant_act_grouped(X, M, K, qx, sxg, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

int aq_decode_split(const aq_packed *W, int M) {
  if (check_packed(W) != AQ_OK || M < 0) return 0;
  return aq::decode_split(aq::view_of(*W), M);
}

size_t aq_workspace_bytes(const aq_packed *W, int M, int phase, int split) {
  if (check_packed(W) != AQ_OK || M <= 0) return 0;
  const aq::PackedView v = aq::view_of(*W);
  if (phase == AQ_PHASE_PREFILL) return aq::prefill_call_workspace_bytes(v, M);
  if (phase == AQ_PHASE_PREFILL_GROUPED)
    return aq::prefill_grouped_long(v, M) ? aq::prefill_workspace_bytes(v, M) : aq::decode_workspace_bytes(v, M, 0);
  if (phase != AQ_PHASE_DECODE && phase != AQ_PHASE_DECODE_TRANSFORMED && phase != AQ_PHASE_DECODE_FP32)
    return 0;
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return 0;
  if (phase == AQ_PHASE_DECODE_FP32) return aq::fp32_workspace_bytes(v, M, split);
  return aq::decode_workspace_bytes(v, M, split, phase == AQ_PHASE_DECODE_TRANSFORMED);
}

aq_status aq_linear_decode(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                           const float *bias, float *Y, int split, void *ws, size_t ws_bytes,
                           void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  const aq::PackedView v = aq::view_of(*W);
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return AQ_ERR_ARG;
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, split), v)) return AQ_ERR_SHAPE;
  st = check_workspace(ws, ws_bytes, aq::decode_workspace_bytes(v, M, split));
  if (st != AQ_OK) return st;
  return aq::launch_decode(v, qx, sx, M, bias, Y, split, ws, nullptr,
                           static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_decode_fp32(const aq_packed *W, const float *X, int M, const float *bias, float *Y,
                                int split, void *ws, size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  if (M < 0) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!X || !Y) return AQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(Y)) return AQ_ERR_ALIGN;
  if (bias && !aligned16(bias)) return AQ_ERR_ALIGN;
  if ((long long)M * W->K > (1LL << 40) || (long long)M * W->N > (1LL << 40) || M > (1 << 30))
    return AQ_ERR_SHAPE;
  const aq::PackedView v = aq::view_of(*W);
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return AQ_ERR_ARG;
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, split), v)) return AQ_ERR_SHAPE;
  st = check_workspace(ws, ws_bytes, aq::fp32_workspace_bytes(v, M, split));
  if (st != AQ_OK) return st;
  return aq::launch_decode_fp32(v, X, M, bias, Y, split, ws, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_decode_noalloc(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                   const float *bias, float *Y, int split, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  const aq::PackedView v = aq::view_of(*W);
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return AQ_ERR_ARG;
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, split), v)) return AQ_ERR_SHAPE;
  const size_t need = aq::decode_workspace_bytes(v, M, split);
  if (need > aq::kDecodeScratchBytes) return AQ_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if (need > 0 && aq::decode_scratch(s, &ws) != hipSuccess) return AQ_ERR_HIP;
  return aq::launch_decode(v, qx, sx, M, bias, Y, split, ws, nullptr, s) == hipSuccess ? AQ_OK
                                                                                        : AQ_ERR_HIP;
}

aq_status aq_linear_decode_grouped(const aq_packed *W, const int8_t *qx, const float *sxg, int M,
                                   const float *bias, float *Y, int split, void *ws, size_t ws_bytes,
                                   void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sxg, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  const aq::PackedView v = aq::view_of(*W);
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return AQ_ERR_ARG;
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, split), v)) return AQ_ERR_SHAPE;
  st = check_workspace(ws, ws_bytes, aq::decode_workspace_bytes(v, M, split));
  if (st != AQ_OK) return st;
  return aq::launch_decode(v, qx, sxg, M, bias, Y, split, ws, nullptr,
                           static_cast<hipStream_t>(stream), true) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_prefill_grouped(const aq_packed *W, const int8_t *qx, const float *sxg, int M,
                                    const float *bias, float *Y, void *ws, size_t ws_bytes,
                                    void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  const aq::PackedView v = aq::view_of(*W);
  if (!aq::prefill_grouped_long(v, M))
    return aq_linear_decode_grouped(W, qx, sxg, M, bias, Y, 0, ws, ws_bytes, stream);
  st = check_linear_io(W, qx, sxg, M, bias, Y);
  if (st != AQ_OK) return st;
  st = check_workspace(ws, ws_bytes, aq::prefill_workspace_bytes(v, M));
  if (st != AQ_OK) return st;
  return run_prefill_grouped(v, qx, sxg, M, bias, Y, nullptr, ws, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_tile_partials_grouped(const aq_packed *W, const int8_t *qx, int M, int32_t *P, void *ws,
                                          size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  if (M < 0) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!qx || !P) return AQ_ERR_NULL;
  if (!aligned16(qx) || !aligned4(P)) return AQ_ERR_ALIGN;
  const aq::PackedView v = aq::view_of(*W);
  if ((long long)M * v.N * (v.K / 64) > (1LL << 40)) return AQ_ERR_SHAPE;
  if (aq::prefill_grouped_long(v, M)) {
    st = check_workspace(ws, ws_bytes, aq::prefill_workspace_bytes(v, M));
    if (st != AQ_OK) return st;
    return run_prefill_grouped(v, qx, nullptr, M, nullptr, nullptr, P, ws, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? AQ_OK
               : AQ_ERR_HIP;
  }
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, 0), v)) return AQ_ERR_SHAPE;
  return aq::launch_decode(v, qx, nullptr, M, nullptr, nullptr, 0, nullptr, P,
                           static_cast<hipStream_t>(stream), true) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_prefill(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                            const float *bias, float *Y, void *ws, size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  const aq::PackedView v = aq::view_of(*W);
  st = check_workspace(ws, ws_bytes, aq::prefill_call_workspace_bytes(v, M));
  if (st != AQ_OK) return st;
  return run_prefill(v, qx, sx, M, bias, Y, nullptr, ws, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_prefill_prepare(const aq_packed *W, void *ws, size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  const aq::PackedView v = aq::view_of(*W);
  const size_t need = aq::prefill_workspace_bytes(v, aq::kLongPrefillM);
  if (need == 0) return AQ_OK;  // no INT4 tile, or no long route: nothing to prepare
  st = check_workspace(ws, ws_bytes, need);
  if (st != AQ_OK) return st;
  const int8_t *E;
  const float *Es;
  return aq::launch_expand(v, ws, static_cast<hipStream_t>(stream), &E, &Es) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_prefill_prepared(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                     const float *bias, float *Y, const void *ws, size_t ws_bytes,
                                     void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  const aq::PackedView v = aq::view_of(*W);
  st = check_workspace(const_cast<void *>(ws), ws_bytes, aq::prefill_workspace_bytes(v, M));
  if (st != AQ_OK) return st;
  return run_prefill(v, qx, sx, M, bias, Y, nullptr, const_cast<void *>(ws),
                     static_cast<hipStream_t>(stream), true) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_tile_partials(const aq_packed *W, const int8_t *qx, int M, int phase,
                                  int32_t *P, void *ws, size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  if (phase != AQ_PHASE_DECODE && phase != AQ_PHASE_PREFILL) return AQ_ERR_ARG;
  if (M < 0) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!qx || !P) return AQ_ERR_NULL;
  if (!aligned16(qx) || !aligned4(P)) return AQ_ERR_ALIGN;
  const aq::PackedView v = aq::view_of(*W);
  if ((long long)M * v.N * v.C > (1LL << 40)) return AQ_ERR_SHAPE;
  if (phase == AQ_PHASE_PREFILL) {
    st = check_workspace(ws, ws_bytes, aq::prefill_workspace_bytes(v, M));
    if (st != AQ_OK) return st;
  } else if (!aq::decode_plan_ok(aq::plan_decode(v, M, 0), v)) {
    return AQ_ERR_SHAPE;
  }
  hipError_t e = phase == AQ_PHASE_DECODE
                     ? aq::launch_decode(v, qx, nullptr, M, nullptr, nullptr, 0, nullptr, P,
                                         static_cast<hipStream_t>(stream))
                     : run_prefill(v, qx, nullptr, M, nullptr, nullptr, P, ws,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AQ_OK : AQ_ERR_HIP;
}

}  // extern "C"

namespace {

// Tables of App. B.1's signed permutations: rows of perm are permutations
// of 0..63, signs are +-1.
aq_status check_tables(const aq_transform_tables *t) {
  if (!t) return AQ_ERR_NULL;
  for (int s = 0; s < AQ_TRANSFORM_SEEDS; ++s) {
    uint64_t seen = 0;
    for (int l = 0; l < 64; ++l) {
      if (t->perm[s][l] >= 64) return AQ_ERR_ARG;
      seen |= 1ull << t->perm[s][l];
      if ((t->dl[s][l] != 1 && t->dl[s][l] != -1) || (t->dr[s][l] != 1 && t->dr[s][l] != -1))
        return AQ_ERR_ARG;
    }
    if (seen != ~0ull) return AQ_ERR_ARG;
  }
  return AQ_OK;
}

aq_status run_row_transform(int kind, const float *src, int M, int K, const int8_t *seeds,
                            const aq_transform_tables *t, const float *bias, float *dst,
                            void *stream) {
  if (M < 0 || K <= 0 || K % 64) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!src || !dst || !seeds) return AQ_ERR_NULL;
  aq_status st = check_tables(t);
  if (st != AQ_OK) return st;
  if (!aligned16(src) || !aligned16(dst) || (bias && !aligned16(bias))) return AQ_ERR_ALIGN;
  if ((long long)M * K > (1LL << 40)) return AQ_ERR_SHAPE;
  return aq::launch_transform(kind, src, dst, M, K, seeds, nullptr, bias, *t,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

}  // namespace

extern "C" {

aq_status aq_transform_rows(const float *X, int M, int K, const int8_t *vseeds,
                            const aq_transform_tables *tables_host, float *Xt, void *stream) {
  return run_row_transform(aq::kTransformRows, X, M, K, vseeds, tables_host, nullptr, Xt, stream);
}

aq_status aq_transform_out(const float *Yt, int M, int N, const int8_t *useeds,
                           const aq_transform_tables *tables_host, const float *bias, float *Y,
                           void *stream) {
  return run_row_transform(aq::kTransformOut, Yt, M, N, useeds, tables_host, bias, Y, stream);
}

aq_status aq_quant_act_transformed(const float *X, int M, int K, const int8_t *vseeds,
                                   const aq_transform_tables *tables_host, int8_t *qx, float *sx,
                                   void *stream) {
  if (M < 0 || K <= 0 || K % 64 || K > aq::kQuantTransformMaxK) return AQ_ERR_SHAPE;
  if (M == 0) return AQ_OK;
  if (!X || !qx || !sx || !vseeds) return AQ_ERR_NULL;
  aq_status st = check_tables(tables_host);
  if (st != AQ_OK) return st;
  if (!aligned16(X) || !aligned16(qx) || !aligned4(sx)) return AQ_ERR_ALIGN;
  if ((long long)M * K > (1LL << 40)) return AQ_ERR_SHAPE;
  return aq::launch_quant_act_transformed(X, M, K, vseeds, *tables_host, qx, sx,
                                          static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_transform_weights(const float *W, int N, int K, const int8_t *useeds,
                               const int8_t *vseeds, const aq_transform_tables *tables_host,
                               float *Wt, void *stream) {
  if (N <= 0 || K <= 0 || N % 64 || K % 64) return AQ_ERR_SHAPE;
  if (!W || !Wt || !useeds || !vseeds) return AQ_ERR_NULL;
  aq_status st = check_tables(tables_host);
  if (st != AQ_OK) return st;
  if (!aligned16(W) || !aligned16(Wt)) return AQ_ERR_ALIGN;
  if ((long long)N * K > (1LL << 40) || N / 64 > 65535) return AQ_ERR_SHAPE;
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(W), t0 = reinterpret_cast<uintptr_t>(Wt);
  const uintptr_t bytes = (uintptr_t)N * K * sizeof(float);
  if (w0 < t0 + bytes && t0 < w0 + bytes) return AQ_ERR_ARG;
  return aq::launch_transform(aq::kTransformWeights, W, Wt, N, K, vseeds, useeds, nullptr, *tables_host,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_decode_transformed(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                       const float *bias, const int8_t *useeds,
                                       const aq_transform_tables *tables_host, float *Y, int split,
                                       void *ws, size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  if (!useeds) return AQ_ERR_NULL;
  st = check_tables(tables_host);
  if (st != AQ_OK) return st;
  const aq::PackedView v = aq::view_of(*W);
  if (split < 0 || (split > 0 && !aq::decode_split_supported(v, M, split))) return AQ_ERR_ARG;
  if (!aq::decode_plan_ok(aq::plan_decode(v, M, split, true), v, true)) return AQ_ERR_SHAPE;
  st = check_workspace(ws, ws_bytes, aq::decode_workspace_bytes(v, M, split, true));
  if (st != AQ_OK) return st;
  return aq::launch_decode_transformed(v, qx, sx, M, bias, Y, split, ws, useeds, *tables_host,
                                       static_cast<hipStream_t>(stream)) == hipSuccess
             ? AQ_OK
             : AQ_ERR_HIP;
}

aq_status aq_linear_prefill_transformed(const aq_packed *W, const int8_t *qx, const float *sx, int M,
                                        const float *bias, const int8_t *useeds,
                                        const aq_transform_tables *tables_host, float *Y, void *ws,
                                        size_t ws_bytes, void *stream) {
  aq_status st = check_packed(W);
  if (st != AQ_OK) return st;
  st = check_linear_io(W, qx, sx, M, bias, Y);
  if (st != AQ_OK || M == 0) return st;
  if (!useeds) return AQ_ERR_NULL;
  st = check_tables(tables_host);
  if (st != AQ_OK) return st;
  const aq::PackedView v = aq::view_of(*W);
  st = check_workspace(ws, ws_bytes, aq::prefill_call_workspace_bytes(v, M));
  if (st != AQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (aq::prefill_long(v, M)) {
    // the long-prompt GEMMs apply U in their epilogue
    const int8_t *E = v.w8;
    const float *Es = v.s8;
    if (v.T4 > 0 && aq::launch_expand(v, ws, s, &E, &Es) != hipSuccess) return AQ_ERR_HIP;
    const hipError_t e = aq::prefill_big_fits(v.N, v.K, v.bK, M)
                             ? aq::launch_prefill_big(E, Es, v.N, v.K, qx, sx, M, bias, Y, nullptr, s, useeds,
                                                      tables_host)
                             : aq::launch_prefill_dense(E, Es, v.N, v.K, v.bK, qx, sx, M, bias, Y, nullptr, s,
                                                        useeds, tables_host);
    return e == hipSuccess ? AQ_OK : AQ_ERR_HIP;
  }
  // short prompts: the decode kernels or the 32 x 32 MFMA GEMM, U in the
  // epilogue of either
  if (aq::prefill_on_decode(v, M, true)) {
    const bool handover = aq::decode_workspace_bytes(v, M, 0, true) > 0;
    if (handover && aq::launch_zero_counters(ws, s) != hipSuccess) return AQ_ERR_HIP;
    return aq::launch_decode_transformed(v, qx, sx, M, bias, Y, 0, handover ? ws : nullptr, useeds,
                                         *tables_host, s) == hipSuccess
               ? AQ_OK
               : AQ_ERR_HIP;
  }
  return aq::launch_prefill(v, qx, sx, M, bias, Y, nullptr, s, useeds, tables_host) == hipSuccess ? AQ_OK
                                                                                                 : AQ_ERR_HIP;
}

}  // extern "C"
