// Host-only planning of the kernels' launches and workspaces: decode work
// split, token groups and column chunks; the long-prompt GEMM's choice of
// kernel; the temporary operand's size.  No device code, so the host side of
// the library (this file and aq_api.cpp) also builds with a plain C++
// compiler, as the sanitizer check in the tests does.

#include <hip/hip_runtime_api.h>

#include "aq_internal.h"

namespace aq {
namespace {

// Packed tiles of more than 16 MB: a projection too large to stay in the
// on-chip caches between calls.
bool streams_from_hbm(const PackedView &w) {
  return (long long)w.T4 * 64 * w.bK / 2 + (long long)w.T8 * 64 * w.bK > (16LL << 20);
}

// Token groups of 16 per workgroup, waves per workgroup, token chunks.  Up
// to 64 tokens share one pass over the weights; on projections that stream
// from HBM, groups of at most 32 tokens (one token chunk after another)
// measure faster at M = 33..128 than 48 or 64 tokens in one pass (8B-class
// gate_up at M = 64: 49.5 us in two chunks of 32, 59.9 us in one pass of 64
// on 16 waves with the columns in two chunks).
int mgroups(const PackedView &w, int M) {
  const int g = M >= 49 ? 4 : (M + 15) / 16;
  return streams_from_hbm(w) && g > 2 ? 2 : g;
}
// 16 waves for every token-group count; 3-4 groups take 4 tiles per batch to
// stay within 128 registers.  Measured on 8B-class qkv and o (M = 48, 64):
// 14.7 / 17.6 us and 13.8 / 16.7 us, against 17.8 / 19.7 and 16.9 / 18.8 us
// with 8 waves and 6 tiles per batch.
int waves_of(const PackedView &w, int M) {
  (void)w;
  (void)M;
  return 16;
}
int mchunks_of(const PackedView &w, int M) {
  const int MG = mgroups(w, M);
  return (M + 16 * MG - 1) / (16 * MG);
}

// LDS row stride of one token's chunk of cz tile columns.
int chunk_stride(int cz, int bK) { return ((cz * bK + 255) / 256) * 256; }

// Bytes of the staged token rows of a chunk of cz columns.
size_t chunk_lds(int MG, int cz, int bK) { return (size_t)16 * MG * chunk_stride(cz, bK); }

// Fewest chunks whose token rows fit in LDS.
int chunks_to_fit(const PackedView &w, int MG) {
  for (int z = 1; z < w.C; ++z)
    if (chunk_lds(MG, (w.C + z - 1) / z, w.bK) <= (size_t)kLdsBudget) return z;
  return w.C;
}

// Row groups per workgroup without chunking: the fewest that still let the
// whole grid (4R/RG workgroups, one per CU at this occupancy) run in a single
// round on the 256 CUs; more row groups per workgroup means fewer, longer
// splits.
int rowgroups_unchunked(const PackedView &w) {
  const int cus = 256;
  if (4 * w.R <= cus) return 1;
  if (2 * w.R <= cus) return 2;
  return 4;
}

// Adaptive row groups and chunks for the shared-activation MFMA path.
// When the tokens' activations over all K fit in LDS the call is not
// chunked (the row-group rule above).  Otherwise the workgroup takes a whole
// 64-row tile row (RG = 4: every staged activation byte feeds 64 weight rows)
// and the columns are cut into the fewest chunks that fit.  Measured on the
// 3B-14B projection shapes at M = 8..64: more chunks (to occupy more CUs)
// lose, since every chunked workgroup adds a serial stage-load-store-count
// chain, and fewer row groups per workgroup lose to the extra activation
// staging.
void choose_chunks(const PackedView &w, int M, int MG, int *RG, int *Z) {
  (void)M;
  const int zfit = chunks_to_fit(w, MG);
  if (zfit == 1) {
    *RG = rowgroups_unchunked(w);
    *Z = 1;
  } else {
    *RG = 4;
    *Z = zfit;
  }
}

}  // namespace

DecodePlan plan_decode(const PackedView &w, int M, int split, bool xform) {
  DecodePlan p;
  p.MG = mgroups(w, M);
  p.waves = waves_of(w, M);
  p.mchunks = mchunks_of(w, M);
  // Products on MFMA for every M (with one token, 15 of the 16 A-operand rows
  // are padding, yet it measured 1-3% faster than the vector-ALU dot
  // products); launch_decode keeps the vector ALU for the one-token grouped
  // route, where it measured about 1% faster.
  p.mode = kMfma;
  p.Z = 1;
  p.ylaunch = p.mchunks;
  p.xstride = 0;
  p.ws_bytes = 0;
  p.cnt_bytes = 0;
  const size_t red = (size_t)p.waves * p.MG * 64 * sizeof(float4);
  // Products: vector ALU for one token, MFMA otherwise.  Activations: a
  // per-wave LDS slice of each batch for M <= 4 (no workgroup barrier),
  // else the block's 16*MG token rows over its chunk of columns.
  p.depth = kPrivDepth;
  // 5..16 tokens: per-wave slices of 4 tiles where each wave's columns are
  // one batch, the workgroup holds one row group (its waves then read
  // disjoint columns) and the staged token rows would be large (M*K of at
  // least 64 KB), instead of the block's staged rows (no workgroup-wide
  // staging before the first products).  Llama-3.2-3B-shaped shapes at
  // M = 16: down (3072 x 8192) 8.74 -> 7.80-7.82 us; o (3072 x 3072, 48 KB of
  // rows) 5.84 -> 5.89-6.03 us and qkv (two row groups per workgroup, whose
  // waves would load the same columns twice) 6.20 -> 6.66 us, so those keep
  // the staged rows.
  const int rg16 = split > 0 ? p.waves / split : rowgroups_unchunked(w);
  const bool priv16 = !xform && w.bK == 128 && M > kPrivMaxM && M <= kPriv16MaxM && rg16 == 1 &&
                      (long long)M * w.K >= 65536 && (w.C + p.waves - 1) / p.waves <= kPriv16Depth;
  if (M <= kPrivMaxM || priv16) {
    p.xmode = kXPriv;
    p.RG = rg16;
    p.depth = priv16 ? kPriv16Depth : kPrivDepth;
    p.lds = (size_t)p.waves * M * p.depth * w.bK + red;
    p.mchunks = 1;
  } else {
    p.xmode = kXShared;
    if (split > 0) {
      p.RG = p.waves / split;
      p.Z = chunks_to_fit(w, p.MG);
    } else {
      choose_chunks(w, M, p.MG, &p.RG, &p.Z);
    }
    const int cz = (w.C + p.Z - 1) / p.Z;
    p.xstride = chunk_stride(cz, w.bK);
    const size_t xb = chunk_lds(p.MG, cz, w.bK);
    p.lds = xb > red ? xb : red;  // the reduction buffer reuses the token rows
    if (p.Z > 1) {
      // counters at a fixed place and size, so that calls of any layout can
      // share one workspace; more token chunks than counters allow take
      // several launches along the token axis
      const int blocks = w.R * 4 / p.RG;
      p.ylaunch = p.mchunks < kDecodeCounters / blocks ? p.mchunks : kDecodeCounters / blocks;
      p.cnt_bytes = (size_t)kDecodeCounters * 4;
      p.ws_bytes = p.cnt_bytes + (size_t)w.R * 4 * p.ylaunch * p.Z * p.MG * 64 * sizeof(float4);
    }
  }
  p.S = p.waves / p.RG;
  if (p.mode == kValu || p.xmode == kXPriv) p.ylaunch = 1;
  if (p.ylaunch > 65535) p.ylaunch = 65535;  // grid y limit
  if (xform) {
    // Keep the tile row in one workgroup (4 row groups, no hand-over) when
    // each wave's share of the row still fits one batch of loads.  Measured
    // on the Llama-3.2-3B-shaped projections at M = 1..16: the hand-over
    // (three device-scope round trips, about 1.7 us) costs more than the
    // slower stream of the fewer, wider workgroups on rows of 24 tile
    // columns (qkv, o: 6.8 / 6.5 us against 7.3 / 7.0 us at M = 1), less on
    // rows of 64 (down: 8.6 against 13.7 us).
    if (split == 0 && p.Z == 1 && p.RG < 4) {
      const int s4 = p.waves / 4;
      const int depth = p.xmode == kXPriv ? p.depth
                        : p.MG == 1       ? kSharedDepth1
                        : p.MG == 2       ? kSharedDepthN
                                          : kSharedDepthW;
      if ((w.C + s4 - 1) / s4 <= depth) {
        p.RG = 4;
        p.S = s4;
      }
    }
    if ((4 / p.RG) * p.Z > 1) {
      // one counter per tile row and token chunk of a launch
      const int cap = kDecodeCounters / w.R;
      if (p.ylaunch > cap) p.ylaunch = cap;
      p.cnt_bytes = (size_t)kDecodeCounters * 4;
      p.ws_bytes = p.cnt_bytes + (size_t)w.R * 4 * p.ylaunch * p.Z * p.MG * 64 * sizeof(float4);
    }
    // a flag word, the transform tables, then the tile row's 64 scaled sums
    // per token
    const size_t ylds = 768 + (size_t)16 * p.MG * 64 * sizeof(float);
    if (p.lds < ylds) p.lds = ylds;
  }
  return p;
}

bool decode_plan_ok(const DecodePlan &p, const PackedView &w, bool xform) {
  if ((long long)w.C * p.Z * p.S >= (1LL << 31)) return false;  // 32-bit split bounds
  if (xform && (4 / p.RG) * p.Z > 1 && w.R > kDecodeCounters) return false;
  return p.Z == 1 || w.R * 4 / p.RG <= kDecodeCounters;
}

int decode_split(const PackedView &w, int M) { return plan_decode(w, M, 0).S; }

bool decode_split_supported(const PackedView &w, int M, int S) {
  const int W = waves_of(w, M);
  return S == W || S == W / 2 || S == W / 4;
}

size_t decode_workspace_bytes(const PackedView &w, int M, int split, bool xform) {
  return plan_decode(w, M, split, xform).ws_bytes;
}

// The fused route keeps the per-token plan's row groups and splits (so its
// sums are those of the plan it replaces, bit for bit) and stages the M
// quantized token rows, then a row of per-wave maxima, in LDS.
DecodePlan plan_decode_fused(const PackedView &w, int M, int split) {
  DecodePlan p = plan_decode(w, M, split);
  p.xmode = kXFused;
  p.depth = kPrivDepth;
  p.MG = 1;
  p.Z = 1;
  p.mchunks = 1;
  p.ylaunch = 1;
  p.xstride = chunk_stride(w.C, w.bK);
  const size_t xb = (size_t)(M + 1) * p.xstride;
  const size_t red = (size_t)p.waves * 64 * sizeof(float4);
  p.lds = xb > red ? xb : red;
  p.cnt_bytes = 0;
  p.ws_bytes = 0;
  return p;
}

bool fused_ok(const PackedView &w, int M, int split) {
  if (M < 1 || M > kFusedMaxM || M > kPrivMaxM || w.C > 128) return false;  // labels from one window
  const DecodePlan p = plan_decode_fused(w, M, split);
  if ((long long)M * w.K > 4LL * 64 * p.waves * kFusedUnits) return false;
  return p.mode == kMfma && p.waves == 16 && p.lds <= (size_t)kLdsBudget && decode_plan_ok(p, w);
}

size_t fp32_head_bytes(const PackedView &w, int M, int split) {
  const size_t dws = decode_workspace_bytes(w, M, split);
  const size_t cnt = (size_t)kDecodeCounters * 4;
  return ((dws > cnt ? dws : cnt) + 255) & ~(size_t)255;
}

size_t fp32_workspace_bytes(const PackedView &w, int M, int split) {
  if (M <= 0 || fused_ok(w, M, split)) return 0;
  return fp32_head_bytes(w, M, split) + (((size_t)M * w.K + 255) & ~(size_t)255) +
         (((size_t)M * sizeof(float) + 255) & ~(size_t)255);
}

// Measured on the 8B-class shapes at M = 96 / 128: qkv 26.4 / 29.5 us on the
// decode kernels against 41.9 / 42.0 us on the GEMM (48 blocks), o 16.8 /
// 18.7 against 41.5 / 41.7, down 47.6 / 50.9 against 125.9 / 126.2; gate_up
// (224 blocks) 72.3 / 88.4 against 46.7 / 47.0 stays on the GEMM.
bool prefill_on_decode(const PackedView &w, int M, bool xform) {
  const bool narrow = M <= kPrefillDecodeNarrowM && 2 * ((w.R + 1) / 2) < compute_units();
  return (M <= kPrefillDecodeMaxM || narrow) && decode_plan_ok(plan_decode(w, M, 0, xform), w, xform);
}

size_t prefill_call_workspace_bytes(const PackedView &w, int M) {
  if (prefill_long(w, M)) return prefill_workspace_bytes(w, M);
  size_t need = 0;
  if (prefill_on_decode(w, M, false)) need = plan_decode(w, M, 0, false).ws_bytes;
  if (prefill_on_decode(w, M, true)) {
    const size_t x = plan_decode(w, M, 0, true).ws_bytes;
    if (x > need) need = x;
  }
  return need;
}

size_t expand_bytes(const PackedView &w) {
  const size_t e = (size_t)w.N * w.K;               // INT8 tiles
  const size_t s = (size_t)w.R * w.C * 64 * 4;      // FP32 scales
  return ((e + 255) & ~(size_t)255) + s;
}

// Compute units of the current device (one persistent workgroup each).
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Taken for wide projections (N >= 6144) with tiles for at least half of
// the compute units.  Its 256 x 256 tiles do about 30% more per CU-second
// than the 256 x 128 kernel: on Qwen3-4B-shaped gate_up at M = 2048 (608
// tiles, 2.4 rounds) it takes 179 us against 192 us for the 256 x 128
// kernel's 4.75 rounds, and on qkv (192 tiles on 256 CUs) 61 us against
// 68 us for two rounds of 256 x 128 blocks; likewise on Qwen3-14B-shaped
// gate_up and qkv at M = 8192.  Narrower projections give too few tiles.
bool prefill_big_fits(int N, int K, int bK, int M) {
  constexpr int kBM = 256, kBK = 128;  // the persistent kernel's tile: 256 tokens x 4 tile rows
  if (bK != kBK || N < 6144) return false;
  const long long tiles = (long long)((M + kBM - 1) / kBM) * ((N / 64 + 3) / 4);
  return K / bK >= 2 && 2 * tiles >= compute_units() && (long long)M * N < (1LL << 29);
}

}  // namespace aq
