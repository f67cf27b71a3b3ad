// Memory-bound phase of the tile-aligned W4/W8 x A8 linear layer
// (AlignQuant Sec. 3.3 "Decode parallelism"; App. E.3, Table 5, eq. 19).
//
// Work distribution: output features x input-column groups (Sec. 3.3).  A
// workgroup of WAVES wavefronts owns RG of the four 16-row groups of one
// 64-row output-tile row r and all of its input-tile columns; its wavefronts
// form RG x S, S = WAVES / RG, and wave (rg, s) streams row group rg over
// split s = input-tile columns floor(C*s/S) .. floor(C*(s+1)/S)-1
// (App. E.3).  The S FP32 partials of a row group are summed through LDS in
// increasing s inside the workgroup, so a call is one kernel launch with no
// cross-workgroup synchronization and no workspace.  RG is chosen per shape
// so that the grid has about one workgroup per CU.
//
// Lane l of a wave owns weight row i16 = l % 16 of its row group and
// k-group g = l / 16 of every tile: 16 bytes of each 1 KB panel row
// (two panels of an INT8 tile at b_K = 128, one of an INT4 tile), so one
// wave-wide 16-byte load streams 256 contiguous bytes per k-group.
//   b_K = 128, INT8: step u, k-group g <- panel 2g+u   (columns 32g+16u ..)
//   b_K = 128, INT4: k-group g <- panel g; low nibbles feed step 0 (32g ..),
//                    high nibbles step 1 (32g+16 ..)
//   b_K =  64, INT8: k-group g <- panel g (columns 16g ..)
//   b_K =  64, INT4: k-group g <- bytes 8(g&1) .. +7 of panel g>>1: low
//                    nibbles columns 32(g>>1)+8(g&1) .., high nibbles +16
// A wave issues the loads of up to DEPTH tiles of its split at once and
// then multiplies them; only tiles of the split are loaded.
//
// Physical tile indices follow eq. 16 (row offset plus the same-precision
// tiles before the column) and are tracked in scalar registers; the labels
// of the row (App. E.1) and both row offsets are fetched with one batch of
// scalar loads.
//
// INT8 activations are staged in LDS with coalesced 16-byte loads:
//   M <= 4 : each wave loads, with every weight batch, the batch's columns of
//            the M tokens (lane l: 16 bytes at column t0*b_K + 16l) into a
//            slice of its own, so no workgroup barrier is needed;
//   M  > 4 : the workgroup stages its 16*MG tokens once (loads issued with
//            the metadata loads; 16-byte granules XOR-swizzled by token row so
//            that the 16 rows one MFMA operand reads fall in distinct banks)
//            and publishes them with one barrier while the first weight batch
//            is in flight; when they do not fit, lanes read them from global
//            memory instead;
//   fused  : (M <= 4, from FP32 activations) the workgroup loads the tokens'
//            FP32 rows right behind its first weight batch, finds each row's
//            max |x| (waves, then LDS, one barrier), quantizes the rows by the
//            rule of the activation quantizer (App. B.3: per-token scale,
//            INT8 codes) into the staged layout above and publishes them with
//            the staging barrier; the rows come from L2 faster than the
//            weights from HBM, so only the quantization itself is added to
//            the critical path, not a second kernel launch.
//
// Products (the pages split decode by M too, Table 5, with byte dot
// products for one token):
//   MFMA  : v_mfma_i32_16x16x64_i8 with up to 16 tokens as the A operand and
//           the 16 weight rows as the B operand, C[token 4g+e][row i16]; for
//           every M of the per-token route, one token included (the padding
//           rows cost the matrix core, not the vector ALU or the memory
//           path, and measured 1-3% faster than the dot products);
//   VALU  : v_dot4_i32_i8 (a 4-way byte dot product) for the one-token
//           grouped route; a lane accumulates its 32 columns per tile and
//           the four k-groups are summed across lanes (swizzle / permute)
//           before the split reduction.
// Each tile's INT32 product is rescaled by its per-row FP32 scale into FP32
// accumulators (eq. 19).  INT4 tiles are widened x16 (see w4_lo16), so their
// scale is multiplied by the exact factor 1/16.

#include <cstring>
#include <mutex>

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_quant.h"

namespace aq {
namespace {

struct DecodeArgs {
  const uint8_t *labels;
  const int32_t *off4, *off8;
  const uint8_t *w4;
  const int8_t *w8;
  const float *s4, *s8;
  const int8_t *qx;
  const float *sx, *bias;
  float *Y;
  int32_t *P;
  const float *xf;  // fused route: FP32 activations [M][K] (qx and sx unused)
  int N, K, R, C, T4, T8, M, label_words;
  // input-column chunks per row block (one workgroup each), the LDS row
  // stride of staged activations, and the workspace of chunked calls:
  // arrival counters [row block][token chunk], then FP32 sums
  // [row group][token chunk][chunk z][MG][64 lanes] float4
  int Z, ychunks, xstride;
  uint32_t *cnt;
  float4 *part;
  int kg64;  // grouped activation scales: 64-feature groups per row (K/64)
};

// With INL each tile row's record of the host metadata image (row_off4[r],
// row_off8[r], then the labels of the row's tiles as 128 bits, LSB first)
// travels inside the kernel arguments.  The record's place depends only on
// the workgroup id, so it is fetched with the other arguments and the first
// weight loads wait for no metadata load of their own.
//   With XF the epilogue applies the output transform of App. B.1 (Y = Y~ U,
// U_r = Phi_{u_r}^T on the 64 outputs of tile row r): the seeds (device, one
// per tile row) and the six signed permutations, perm bytes and sign masks
// (bit e set: element e negated), also in the kernel arguments, which leaves
// room for the metadata of fewer tile rows.
struct XfTables {
  uint8_t perm[kTransformSeeds][64];
  uint64_t dlm[kTransformSeeds], drm[kTransformSeeds];
};
constexpr int kXfWords = sizeof(XfTables) / 4;
// staged in 512 bytes of LDS, one word per thread
static_assert(sizeof(XfTables) % 4 == 0 && sizeof(XfTables) <= 512, "transform tables");
struct XfArgs {
  const int8_t *useeds;
  XfTables xt;
};
template <bool INL, bool XF> struct DArgs : DecodeArgs {};
template <> struct DArgs<true, false> : DecodeArgs { uint32_t meta[kInlineWords]; };
template <> struct DArgs<false, true> : DecodeArgs { XfArgs xf; };
template <> struct DArgs<true, true> : DecodeArgs {
  XfArgs xf;
  uint32_t meta[kInlineWordsXf];
};
static_assert(sizeof(DArgs<true, false>) <= 4096 && sizeof(DArgs<true, true>) <= 4096,
              "kernel arguments exceed 4 KiB");

// H_64 over the wave for the output transform, lane l holding element l,
// in the order h = 1, 2, .., 32 (the lane with bit h clear keeps self +
// partner, its partner partner - self), then the exact 1/8: the FP32
// sequence of the separate output transform.  Partners through DPP quad
// permutes (h = 1, 2), ds_swizzle in bit-mask mode (h = 4, 8, 16) and
// ds_bpermute (h = 32).
template <int CTRL>
__device__ __forceinline__ float xf_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int PAT>
__device__ __forceinline__ float xf_swz(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PAT));
}
__device__ __forceinline__ float xf_fwht64(float v, int lane) {
  float p = xf_dpp<0xB1>(v);  // lane ^ 1
  v = (lane & 1) ? p - v : v + p;
  p = xf_dpp<0x4E>(v);  // lane ^ 2
  v = (lane & 2) ? p - v : v + p;
  p = xf_swz<0x101F>(v);  // lane ^ 4
  v = (lane & 4) ? p - v : v + p;
  p = xf_swz<0x201F>(v);  // lane ^ 8
  v = (lane & 8) ? p - v : v + p;
  p = xf_swz<0x401F>(v);  // lane ^ 16
  v = (lane & 16) ? p - v : v + p;
  p = __shfl_xor(v, 32);
  v = (lane & 32) ? p - v : v + p;
  return v * 0.125f;
}

__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

// Weight panels: with NT the loads are non-temporal, so that a projection
// streamed once per call does not evict what the caches hold for others.
template <bool NT>
__device__ __forceinline__ v4i wload16(const void *p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
  else return load16(p);
}
template <bool NT>
__device__ __forceinline__ uint2 wload8(const void *p) {
  if constexpr (NT) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2 *>(p);
  }
}

// Device-coherent FP32x4 store / load (agent-scope relaxed atomics, one per
// element): visible across the whole GPU without cache maintenance.
__device__ __forceinline__ void store_coherent(float4 *p, float4 v) {
  float *q = reinterpret_cast<float *>(p);
  __hip_atomic_store(q + 0, v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 2, v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 3, v.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load_coherent(const float4 *p) {
  const float *q = reinterpret_cast<const float *>(p);
  return make_float4(__hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint2 load8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }

// Labels of tiles tb .. tb+127 (bit k = tile tb + k) from five whole words
// w[0..4] = label words tb/32 .. tb/32+4 (indices clamped into the padded
// buffer: bits beyond the tile row are never read).
__device__ __forceinline__ void label_window(const uint32_t (&w)[5], int tb, uint64_t &lo, uint64_t &hi) {
  const int sh = tb & 31;
  const uint64_t x0 = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  const uint64_t x1 = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
  const uint64_t x2 = (uint64_t)w[4];
  lo = sh ? (x0 >> sh) | (x1 << (64 - sh)) : x0;
  hi = sh ? (x1 >> sh) | (x2 << (64 - sh)) : x1;
}

// Bits s .. s+63 of the 128-bit window (hi:lo); zero from bit 128 on.
__device__ __forceinline__ uint64_t window_bits(uint64_t lo, uint64_t hi, int s) {
  if (s == 0) return lo;
  if (s < 64) return (lo >> s) | (hi << (64 - s));
  if (s < 128) return hi >> (s - 64);
  return 0;
}

__device__ __forceinline__ uint64_t low_mask(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

// Sum over the four k-groups (lanes i16, i16+16, i16+32, i16+48).  Every
// lane ends with the same value: FP32 addition is commutative, and each
// lane adds the same pairs.
__device__ __forceinline__ float sum_kgroups(float v) {
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ int sum_kgroups_i(int v) {
  v += __builtin_amdgcn_ds_swizzle(v, 0x401F);
  v += __shfl_xor(v, 32);
  return v;
}

// 16-byte activation operand of step u for a lane of k-group g, from a row
// of INT8 activations whose column colbase is the tile's first column.  For
// b_K = 64 INT4 tiles the operand is two 8-byte pieces (low-nibble and
// high-nibble columns).  With SW >= 0 the row is an LDS row whose 16-byte
// granules are XOR-swizzled by SW.
template <int BK, bool GRP>
__device__ __forceinline__ v4i x_operand(const int8_t *row, int colbase, int g, int u, int is4, int sw) {
  if (BK == 128 && GRP) {  // step u = 64-feature group u of the tile
    const int c = colbase + 64 * u + 16 * g;
    return load16(row + 16 * ((c >> 4) ^ sw));
  }
  if (BK == 64 && is4) {
    const int ca = colbase + 32 * (g >> 1) + 8 * (g & 1);
    const int cb = ca + 16;
    const uint2 p0 = load8(row + 16 * ((ca >> 4) ^ sw) + (ca & 15));
    const uint2 p1 = load8(row + 16 * ((cb >> 4) ^ sw) + (cb & 15));
    return v4i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y};
  }
  const int c = BK == 128 ? colbase + 32 * g + 16 * u : colbase + 16 * g;
  return load16(row + 16 * ((c >> 4) ^ sw));
}

template <int BK, int MODE, int MG, int WAVES, int RG, int DEPTH, int XMODE, bool PARTIALS, bool INL,
          bool GRP, bool WNT, bool XF>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(const DArgs<INL, XF> a) {
  static_assert(!XF || (MODE == kMfma && !PARTIALS && !GRP), "output transform: per-token MFMA route");
  static_assert(!XF || WAVES * 64 >= kXfWords, "one transform-table word per thread");
  constexpr int KS = BK / 64;    // MFMA steps (16-byte operands per lane) per tile
  constexpr int S = WAVES / RG;  // splits per row group
  constexpr int NT = WAVES * 64;
  constexpr int XU = 8;          // activation granules per thread per staging pass
  constexpr int XW = DEPTH * BK; // bytes of one token's activations per batch (per-wave slices)
  // Per-wave slices of 4 tiles hold up to 16 tokens: each slot of a lane
  // carries one 16-byte granule of XTPS tokens (XLPT lanes per token); the
  // 8-tile slices keep one token per slot, lane l at granule l.
  constexpr bool P16 = XMODE == kXPriv && DEPTH == kPriv16Depth;
  constexpr int XLPT = P16 ? XW / 16 : 64;
  constexpr int XTPS = P16 ? 64 / XLPT : 1;
  constexpr int XSLOTS = P16 ? kPriv16MaxM / XTPS : kPrivMaxM;
  static_assert(!P16 || (BK == 128 && XLPT * XTPS == 64), "16-token slices: b_K = 128");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blocks_per_row = 4 / RG;
  const int Z = a.Z;
  const int zc = blockIdx.z;  // input-column chunk of this workgroup
  const int yc = blockIdx.y;  // token chunk
  const int bx = blockIdx.x;  // row block
  const int Y = gridDim.y;    // token chunks of this launch
  const int r = bx / blocks_per_row;
  const int rgl = wave % RG;  // row group inside the block
  const int rg = (bx % blocks_per_row) * RG + rgl;
  const int sp = wave / RG;   // split of this wave inside the workgroup
  // the row's metadata record when it travels in the kernel arguments; its
  // place depends on the workgroup id alone, so these loads go out with the
  // first argument loads
  uint32_t rec[kMetaStride];
  if constexpr (INL) {
#pragma unroll
    for (int k = 0; k < kMetaStride; ++k) rec[k] = a.meta[kMetaStride * r + k];
    // everything the first weight loads need, fetched in that same batch
    // (the compiler would otherwise load these after the first wait)
    asm volatile("" ::"s"(a.w4), "s"(a.w8), "s"(a.s4), "s"(a.s8), "s"(a.qx), "s"(a.T4), "s"(a.T8),
                 "s"(a.C), "s"(a.K), "s"(a.M), "s"(a.Z));
  }
  // the tile row's output-transform seed, loaded with the metadata
  int useed = 0;
  if constexpr (XF) useed = a.xf.useeds[r];
  const int C = a.C, K = a.K, M = a.M;
  // global split zc*S + sp of Z*S: tile columns floor(C*s/(Z*S)) .. (the
  // planner keeps C*Z*S below 2^31; one chunk: S is a compile-time divisor)
  int ca, c0, c1;
  if (Z == 1) {
    ca = 0;
    c0 = (C * sp) / S;
    c1 = (C * (sp + 1)) / S;
  } else {
    const unsigned ST = (unsigned)(Z * S);
    ca = (int)((unsigned)(C * zc) / (unsigned)Z);  // first column of the chunk
    c0 = (int)((unsigned)(C * (zc * S + sp)) / ST);
    c1 = (int)((unsigned)(C * (zc * S + sp + 1)) / ST);
  }
  const int mbase = yc * 16 * MG;
  const int xrows = MODE == kValu ? M : min(M - mbase, 16 * MG);  // token rows of this block
  const int g = lane >> 4, i16 = lane & 15;
  const int rowoff = rg * 256 + i16 * 16;  // this lane's row inside a 1 KB panel
  const uint8_t *__restrict__ w4p = a.w4;
  const uint8_t *__restrict__ w8p = reinterpret_cast<const uint8_t *>(a.w8);
  const int T4 = a.T4, T8 = a.T8;
  // Staged activations: the chunk's columns ca*BK .. cb*BK of each token row,
  // kg 16-byte granules, at a row stride (xstride) that is a multiple of
  // 256 bytes, granule q of row t stored at q ^ (t & 15): the 16 token rows
  // one MFMA operand reads fall in distinct banks.
  const int cb = Z == 1 ? C : (int)((unsigned)(C * (zc + 1)) / (unsigned)Z);
  const int kg = (cb - ca) * (BK / 16);
  const int xst = a.xstride;
  // LDS: per-wave slices [WAVES][M][DEPTH*BK], or the block's [16*MG] token
  // rows; the split reduction buffer [WAVES][MG][64] float4 follows the
  // slices and reuses the token rows once every wave is done with them.
  int8_t *xs = reinterpret_cast<int8_t *>(smem);
  int8_t *xw = xs + wave * M * XW;
  float4 *red = reinterpret_cast<float4 *>(smem + (XMODE == kXPriv ? WAVES * M * XW : 0));

  // ---- MFMA path: block activation staging loads (independent of the
  // metadata), issued first
  v4i xb[XU];
  const int8_t *xsrc = a.qx + (size_t)mbase * K + (size_t)ca * BK;
  const bool xstage = XMODE == kXShared;
  constexpr bool FUSED = XMODE == kXFused;
  const int xgran = xstage ? xrows * kg : 0;
  if (xstage) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      if (u * NT < xgran) {  // uniform: only the passes the block needs
        const int q = min(tid + u * NT, xgran - 1);
        const int row = q / kg, cg = q - row * kg;
        xb[u] = load16(xsrc + (size_t)row * K + 16 * cg);
      }
    }
  }

  // ---- eq. 16 bookkeeping: the row's offsets and label words in one batch
  // of scalar loads.  The label window below depends on the offsets (a
  // guard that valid metadata never trips), so the compiler cannot defer the
  // offset loads to their later use: all seven share one wait.
  const int tb = r * C;
  const bool fastlab = INL || C <= 128;  // the inline record holds the whole row
  int o4, o8;
  uint64_t wlo, whi;
  if constexpr (INL) {
    // the row's record (loaded above): offsets, then its labels
    o4 = (int)rec[0];
    o8 = (int)rec[1];
    wlo = (uint64_t)rec[2] | ((uint64_t)rec[3] << 32);
    whi = (uint64_t)rec[4] | ((uint64_t)rec[5] << 32);
  } else {
    uint32_t lw[5];
    const int w0 = tb >> 5, last = a.label_words - 1;
    o4 = a.off4[r];
    o8 = a.off8[r];
    const uint32_t *wd = reinterpret_cast<const uint32_t *>(a.labels);
#pragma unroll
    for (int k = 0; k < 5; ++k) lw[k] = wd[min(w0 + k, last)];
    if ((o4 | o8) < 0) lw[4] = 0u;  // negative row offsets: inconsistent metadata
    label_window(lw, tb, wlo, whi);
  }
  int n4 = c0 <= 64 ? __popcll(wlo & low_mask(c0)) : __popcll(wlo) + __popcll(whi & low_mask(c0 - 64));
  int idx4 = o4 + n4;
  int idx8 = o8 + (c0 - n4);
  if (!fastlab) {  // rows of more than 128 tiles: count from memory
    n4 = count_int4(a.labels, tb, c0, a.label_words);
    idx4 = o4 + n4;
    idx8 = o8 + (c0 - n4);
  }

  float4 F[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) F[mg] = make_float4(0.f, 0.f, 0.f, 0.f);

  v4i W[DEPTH][2];
  float SC[DEPTH];
  int live[DEPTH], is4v[DEPTH], jv[DEPTH];
  v4i xv[XSLOTS];  // per-wave slices: this lane's granules of the batch

  // Issue the loads of the live tiles among t0 .. t0+DEPTH-1 of the split:
  // the rows' 16-byte panel chunks (two for an INT8 tile at b_K = 128, one
  // otherwise) and the lane's row scale; with per-wave slices also the
  // batch's activation columns (lane l: 16 bytes at column t0*BK + 16l of
  // each token).  Live tiles are a prefix; the branches are uniform.
#define AQ_DECODE_ISSUE(t0_)                                                                    \
  {                                                                                             \
    const int t0i = (t0_);                                                                      \
    const uint32_t labs = fastlab ? (uint32_t)window_bits(wlo, whi, t0i)                        \
                                  : label_bits32(a.labels, tb + t0i, a.label_words);            \
    _Pragma("unroll") for (int d = 0; d < DEPTH; ++d) {                                         \
      const int jt = t0i + d;                                                                   \
      live[d] = 0;                                                                              \
      if (jt < c1) {                                                                            \
        const int is4 = (int)(labs >> d) & 1;                                                   \
        const int idx = is4 ? idx4 : idx8;                                                      \
        idx4 += is4;                                                                            \
        idx8 += is4 ^ 1;                                                                        \
        /* inconsistent metadata: no valid tile at this index, skip it */                       \
        if (is4 ? (idx >= 0 && idx < T4) : (idx >= 0 && idx < T8)) {                            \
          live[d] = 1;                                                                          \
          is4v[d] = is4;                                                                        \
          jv[d] = jt;                                                                           \
          if (BK == 128 && GRP) {                                                               \
            /* step u: columns 64u + 16g ..: INT8 panel 4u + g; INT4 panel */                   \
            /* 2u + g/2, nibble g % 2 */                                                         \
            if (is4) {                                                                          \
              const uint8_t *base = w4p + (size_t)idx * 4096 + (g >> 1) * 1024 + rowoff;        \
              W[d][0] = wload16<WNT>(base);                                                           \
              W[d][1] = wload16<WNT>(base + 2048);                                                    \
            } else {                                                                            \
              const uint8_t *base = w8p + (size_t)idx * 8192 + g * 1024 + rowoff;               \
              W[d][0] = wload16<WNT>(base);                                                           \
              W[d][1] = wload16<WNT>(base + 4096);                                                    \
            }                                                                                   \
          } else if (BK == 128) {                                                               \
            if (is4) {                                                                          \
              W[d][0] = wload16<WNT>(w4p + (size_t)idx * 4096 + g * 1024 + rowoff);                   \
            } else {                                                                            \
              const uint8_t *base = w8p + (size_t)idx * 8192 + (2 * g) * 1024 + rowoff;         \
              W[d][0] = wload16<WNT>(base);                                                           \
              W[d][1] = wload16<WNT>(base + 1024);                                                    \
            }                                                                                   \
          } else {                                                                              \
            if (is4) {                                                                          \
              const uint2 lo = wload8<WNT>(w4p + (size_t)idx * 2048 + (g >> 1) * 1024 + rowoff + 8 * (g & 1)); \
              W[d][0] = v4i{(int)lo.x, (int)lo.y, 0, 0};                                        \
            } else {                                                                            \
              W[d][0] = wload16<WNT>(w8p + (size_t)idx * 4096 + g * 1024 + rowoff);                   \
            }                                                                                   \
          }                                                                                     \
          SC[d] = (is4 ? a.s4 : a.s8)[(size_t)idx * 64 + rg * 16 + i16];                        \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
    if (XMODE == kXPriv && P16) {                                                               \
      const int col = min(t0i * BK + 16 * (lane % XLPT), K - 16);                               \
      _Pragma("unroll") for (int q = 0; q < XSLOTS; ++q) {                                      \
        const int m = q * XTPS + lane / XLPT;                                                   \
        if (m < M) xv[q] = load16(a.qx + (size_t)m * K + col);                                  \
      }                                                                                         \
    } else if (XMODE == kXPriv) {                                                               \
      const int col = min(t0i * BK + 16 * lane, K - 16);                                        \
      _Pragma("unroll") for (int m = 0; m < kPrivMaxM; ++m)                                     \
        if (m < M) xv[m] = load16(a.qx + (size_t)m * K + col);                                  \
    }                                                                                           \
  }

  // ---- MFMA path: block activations into LDS (the stores wait for the
  // staging loads only), then the first weight batch, then one barrier
  // while that batch is in flight
  if (xstage) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int q = tid + u * NT;
      if (u * NT < xgran && q < xgran) {
        const int row = q / kg, cg = q - row * kg;
        *reinterpret_cast<v4i *>(xs + row * xst + 16 * (cg ^ (row & 15))) = xb[u];
      }
    }
    for (int q0 = XU * NT; q0 < xgran; q0 += XU * NT) {  // large blocks only
      v4i xt[XU];
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int q = min(q0 + tid + u * NT, xgran - 1);
        const int row = q / kg, cg = q - row * kg;
        xt[u] = load16(xsrc + (size_t)row * K + 16 * cg);
      }
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int q = q0 + tid + u * NT;
        if (q < xgran) {
          const int row = q / kg, cg = q - row * kg;
          *reinterpret_cast<v4i *>(xs + row * xst + 16 * (cg ^ (row & 15))) = xt[u];
        }
      }
    }
  }
  AQ_DECODE_ISSUE(c0);
  // Epilogue operands, issued behind the first weight batch so that their
  // latency hides under the weight stream: the token scales of the lane's
  // outputs and its bias (with XF the tile row's 64 bias values, one per
  // lane, and the lane's part of the tile row's transform).
  float sxv[MG][4];
  float bv = 0.0f;
  uint32_t xtw = 0u;  // XF: word tid of the transform tables
  if constexpr (!PARTIALS && !GRP && MODE == kMfma) {
    if constexpr (!FUSED) {
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mbase + mg * 16 + 4 * g + e;
          sxv[mg][e] = m < M ? a.sx[m] : 0.0f;
        }
    }
    if (a.bias) bv = a.bias[(size_t)r * 64 + (XF ? lane : rg * 16 + i16)];
  }
  if constexpr (XF) {
    if (tid < kXfWords) xtw = reinterpret_cast<const uint32_t *>(&a.xf.xt)[tid];
  }
  // ---- fused route: the tokens' FP32 rows, kFusedUnits float4 per thread
  // (consecutive threads, consecutive float4), loaded right behind the first
  // weight batch: waiting for them waits for that batch too, whose HBM
  // latency exceeds theirs, so the quantization below starts about when the
  // weights land
  float4 xq32[FUSED ? kFusedUnits : 1];
  const int nf4 = FUSED ? M * (K >> 2) : 0;
  if constexpr (FUSED) {
    // (threads past the rows in a partly used pass re-read a unit inside
    // them, spread over the largest power-of-two prefix: one address read
    // by every workgroup would queue on one L2 channel)
    const float4 *xsrc32 = reinterpret_cast<const float4 *>(a.xf);
    const int p2m = (1 << (31 - __builtin_clz(nf4))) - 1;
#pragma unroll
    for (int u = 0; u < kFusedUnits; ++u) {
      const int q = tid + u * NT;
      if (u * NT < nf4) xq32[u] = xsrc32[q < nf4 ? q : (q & p2m)];
    }
  }
  if constexpr (FUSED) {
    // Per-token quantization, the rule of the activation quantizer: s =
    // max(max|x| / 127, 1e-12) in FP64, codes rint(x / s) clipped to INT8.
    // Row maxima of this thread's units, of the wave (uniform), then of the
    // workgroup through LDS row M of the staging area (the token rows are
    // rows 0 .. M-1).
    const int k4 = K >> 2;
    // token row of unit q without a division (M <= 4)
    auto row_of = [&](int q) __attribute__((always_inline)) {
      return (int)(q >= k4) + (int)(q >= 2 * k4) + (int)(q >= 3 * k4);
    };
    uint32_t pm[kFusedMaxM] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kFusedUnits; ++u) {
      const int q = tid + u * NT;
      if (u * NT < nf4 && q < nf4) {
        const int row = row_of(q);
        const uint32_t v = abs_bits4(xq32[u]);
#pragma unroll
        for (int t = 0; t < kFusedMaxM; ++t)
          if (row == t) pm[t] = max(pm[t], v);
      }
    }
    uint32_t *amx = reinterpret_cast<uint32_t *>(xs + (size_t)M * xst);  // [token][wave]
#pragma unroll
    for (int t = 0; t < kFusedMaxM; ++t) {
      if (t < M) {  // uniform
        const uint32_t v = wave_max_u32(pm[t]);
        if (lane == 0) amx[t * WAVES + wave] = v;
      }
    }
    __syncthreads();
    // lane t < M finds token t's scale and its FP32 reciprocal (one FP64
    // division pair per wave), then every lane takes them from there
    uint32_t mx = 0u;
    if (lane < M) {
      const uint4 *am4 = reinterpret_cast<const uint4 *>(amx + lane * WAVES);
      uint4 v[WAVES / 4];
#pragma unroll
      for (int w4 = 0; w4 < WAVES / 4; ++w4) v[w4] = am4[w4];  // all issued, then one wait
#pragma unroll
      for (int w4 = 0; w4 < WAVES / 4; ++w4) mx = max(mx, max(max(v[w4].x, v[w4].y), max(v[w4].z, v[w4].w)));
    }
    const double sl = row_scale(mx);
    const float il = (float)(1.0 / sl);
    const long long slb = __double_as_longlong(sl);
    double sd[kFusedMaxM];
    float inv[kFusedMaxM], sq[kFusedMaxM];
#pragma unroll
    for (int t = 0; t < kFusedMaxM; ++t) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)slb, t);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(slb >> 32), t);
      sd[t] = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
      inv[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(il), t));
      sq[t] = (float)sd[t];
    }
    // this thread's codes into the token rows, granules swizzled as staged
#pragma unroll
    for (int u = 0; u < kFusedUnits; ++u) {
      const int q = tid + u * NT;
      if (u * NT < nf4 && q < nf4) {
        const int row = row_of(q);
        const int c = (q - row * k4) * 4;
        double sr = sd[0];
        float ir = inv[0];
#pragma unroll
        for (int t = 1; t < kFusedMaxM; ++t)
          if (row == t) {
            sr = sd[t];
            ir = inv[t];
          }
        *reinterpret_cast<uint32_t *>(xs + row * xst + 16 * ((c >> 4) ^ (row & 15)) + (c & 15)) =
            codes4_fast(xq32[u], sr, ir);
      }
    }
    // the token scales of the lane's outputs (one token group)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * g + e;
      float v = 0.0f;
#pragma unroll
      for (int t = 0; t < kFusedMaxM; ++t)
        if (m == t && t < M) v = sq[t];
      sxv[0][e] = v;
    }
  }
  if (xstage || FUSED) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS writes done; vmcnt left open
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  for (int t0 = c0; t0 < c1; t0 += DEPTH) {
    if (t0 != c0) AQ_DECODE_ISSUE(t0);
    if (XMODE == kXPriv && P16) {  // the wave's own activation slice; read back by this wave only
#pragma unroll
      for (int q = 0; q < XSLOTS; ++q) {
        const int m = q * XTPS + lane / XLPT;
        if (m < M) *reinterpret_cast<v4i *>(xw + m * XW + 16 * (lane % XLPT)) = xv[q];
      }
    } else if (XMODE == kXPriv) {
#pragma unroll
      for (int m = 0; m < kPrivMaxM; ++m)
        if (m < M && 16 * lane < XW) *reinterpret_cast<v4i *>(xw + m * XW + 16 * lane) = xv[m];
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (!live[d]) continue;
      const int jt = jv[d];
      const int is4 = is4v[d];
      // weight operand per step
      v4i wop[KS];
      if (BK == 128 && GRP) {
        if (is4) {  // this lane's nibble of both panels
          const v4i w0 = W[d][0], w1 = W[d][1];
          const bool hi = (g & 1) != 0;
          wop[0] = hi ? v4i{w4_hi16(w0[0]), w4_hi16(w0[1]), w4_hi16(w0[2]), w4_hi16(w0[3])}
                      : v4i{w4_lo16(w0[0]), w4_lo16(w0[1]), w4_lo16(w0[2]), w4_lo16(w0[3])};
          wop[KS - 1] = hi ? v4i{w4_hi16(w1[0]), w4_hi16(w1[1]), w4_hi16(w1[2]), w4_hi16(w1[3])}
                           : v4i{w4_lo16(w1[0]), w4_lo16(w1[1]), w4_lo16(w1[2]), w4_lo16(w1[3])};
        } else {
          wop[0] = W[d][0];
          wop[KS - 1] = W[d][1];
        }
      } else if (BK == 128) {
        if (is4) {
          const v4i w = W[d][0];
          wop[0] = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_lo16(w[2]), w4_lo16(w[3])};
          wop[KS - 1] = v4i{w4_hi16(w[0]), w4_hi16(w[1]), w4_hi16(w[2]), w4_hi16(w[3])};
        } else {
          wop[0] = W[d][0];
          wop[KS - 1] = W[d][1];
        }
      } else {
        const v4i w = W[d][0];
        wop[0] = is4 ? v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_hi16(w[0]), w4_hi16(w[1])} : w;
      }
      const float sc = is4 ? SC[d] * 0.0625f : SC[d];
      if (MODE == kMfma) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          // token row of this lane; padding tokens read the last real row,
          // their outputs are never stored
          const int trow = min(mg * 16 + i16, xrows - 1);
          const int8_t *xr = XMODE == kXPriv ? xw + trow * XW : xs + trow * xst;
          const int xcol = XMODE == kXPriv ? d * BK : (jt - ca) * BK;
          const int sw = XMODE != kXPriv ? (trow & 15) : 0;
          if constexpr (GRP) {
            // one INT32 product per 64-feature group (step u), each scaled by
            // its own activation-group scale (token group of 16 rows)
            v4i accg[KS];
#pragma unroll
            for (int u = 0; u < KS; ++u) {
              const v4i xop = x_operand<BK, GRP>(xr, xcol, g, u, is4, sw);
              accg[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xop, wop[u], v4i{0, 0, 0, 0}, 0, 0, 0);
            }
            if constexpr (PARTIALS) {
              const size_t n = (size_t)r * 64 + rg * 16 + i16;
#pragma unroll
              for (int u = 0; u < KS; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int m = mbase + mg * 16 + 4 * g + e;
                  if (m < M)
                    a.P[((size_t)m * a.N + n) * a.kg64 + jt * KS + u] = is4 ? (accg[u][e] >> 4) : accg[u][e];
                }
            } else {
              // a group of padding tokens only (never stored) reads the last
              // real group's scales
              const int grp = min(mbase / 16 + mg, (M - 1) / 16);
              const float *sxr = a.sx + (size_t)grp * a.kg64 + jt * KS;
#pragma unroll
              for (int u = 0; u < KS; ++u) {
                const float c = sc * sxr[u];
                F[mg].x = fmaf((float)accg[u][0], c, F[mg].x);
                F[mg].y = fmaf((float)accg[u][1], c, F[mg].y);
                F[mg].z = fmaf((float)accg[u][2], c, F[mg].z);
                F[mg].w = fmaf((float)accg[u][3], c, F[mg].w);
              }
            }
            continue;
          }
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const v4i xop = x_operand<BK, GRP>(xr, xcol, g, u, is4, sw);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(xop, wop[u], acc, 0, 0, 0);
          }
          if constexpr (PARTIALS) {
            // lane holds tokens mbase + 16mg + 4g + e of row 64r + 16rg + i16
            const size_t n = (size_t)r * 64 + rg * 16 + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = mbase + mg * 16 + 4 * g + e;
              if (m < M) a.P[((size_t)m * a.N + n) * C + jt] = is4 ? (acc[e] >> 4) : acc[e];
            }
          } else {
            F[mg].x = fmaf((float)acc[0], sc, F[mg].x);
            F[mg].y = fmaf((float)acc[1], sc, F[mg].y);
            F[mg].z = fmaf((float)acc[2], sc, F[mg].z);
            F[mg].w = fmaf((float)acc[3], sc, F[mg].w);
          }
        }
      } else if constexpr (GRP) {
        // vector ALU, one token (its own row group): one product per
        // 64-feature group (step u)
        int accg[KS];
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          accg[u] = 0;
          const v4i xop = x_operand<BK, GRP>(xw, d * BK, g, u, is4, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) accg[u] = __builtin_amdgcn_sdot4(wop[u][e], xop[e], accg[u], false);
        }
        if constexpr (PARTIALS) {
          const size_t n = (size_t)r * 64 + rg * 16 + i16;
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const int v = sum_kgroups_i(accg[u]);
            if (g == 0) a.P[n * a.kg64 + jt * KS + u] = is4 ? (v >> 4) : v;
          }
        } else {
#pragma unroll
          for (int u = 0; u < KS; ++u) F[0].x = fmaf((float)accg[u], sc * a.sx[jt * KS + u], F[0].x);
        }
      } else {
        // vector ALU: the one token, this lane's 16*KS columns
        int acc[kValuMaxM];
#pragma unroll
        for (int m = 0; m < kValuMaxM; ++m) {
          acc[m] = 0;
          if (m < M) {
#pragma unroll
            for (int u = 0; u < KS; ++u) {
              const v4i xop = x_operand<BK, GRP>(xw + m * XW, d * BK, g, u, is4, 0);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[m] = __builtin_amdgcn_sdot4(wop[u][e], xop[e], acc[m], false);
            }
          }
        }
        if constexpr (PARTIALS) {
          const size_t n = (size_t)r * 64 + rg * 16 + i16;
#pragma unroll
          for (int m = 0; m < kValuMaxM; ++m) {
            if (m < M) {
              const int v = sum_kgroups_i(acc[m]);
              if (g == 0) a.P[((size_t)m * a.N + n) * C + jt] = is4 ? (v >> 4) : v;
            }
          }
        } else {
          F[0].x = fmaf((float)acc[0], sc, F[0].x);
        }
      }
    }
  }
#undef AQ_DECODE_ISSUE

  if constexpr (!PARTIALS) {
    if (MODE == kValu) F[0].x = sum_kgroups(F[0].x);  // sum the four k-groups of each row
    // ordered split reduction through LDS
    if (S > 1) {
      if (XMODE != kXPriv) __syncthreads();  // every wave is done with the token rows
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) red[(wave * MG + mg) * 64 + lane] = F[mg];
      __syncthreads();
      if (sp == 0) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          float4 v = red[(rgl * MG + mg) * 64 + lane];
#pragma unroll 4
          for (int ss = 1; ss < S; ++ss) {
            const float4 p = red[((ss * RG + rgl) * MG + mg) * 64 + lane];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
          }
          F[mg] = v;
        }
      }
    }
    if constexpr (XF) {
      // Output transform (App. B.1 eq. 4) after the ordered split sum (App.
      // E.3): per tile row, Y = (sx * Y~) U + bias, the token scale applied
      // first so that the result is bit for bit that of the linear followed
      // by the separate output transform.  U mixes the 64 outputs of a tile
      // row.  When its row groups or column chunks ran in several
      // workgroups, each workgroup's sums go to the workspace (slot zc of
      // each of its row groups, device-coherent as for chunked K) and the
      // last workgroup of the tile row to arrive (arrival counter per tile
      // row and token chunk, reset by that workgroup) adds every row
      // group's slots in increasing zc and finishes the tile row.
      uint32_t *flag = reinterpret_cast<uint32_t *>(smem);
      uint32_t *xtl = reinterpret_cast<uint32_t *>(smem + 256);  // the transform tables
      float *ys = reinterpret_cast<float *>(smem + 768);         // [16*MG tokens][64 outputs]
      constexpr int kParts = 4 / RG;                      // workgroups per tile row and chunk
      if (kParts * Z > 1) {
        float4 *pp = a.part + ((size_t)(r * 4 + rg) * Y + yc) * Z * MG * 64 + lane;
        if (sp == 0) {
#pragma unroll
          for (int mg = 0; mg < MG; ++mg) store_coherent(pp + ((size_t)zc * MG + mg) * 64, F[mg]);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if (tid == 0) {
          uint32_t *cp = a.cnt + (size_t)r * Y + yc;
          const uint32_t prev = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t last = prev == (uint32_t)(kParts * Z - 1) ? 1u : 0u;
          if (last) __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          *flag = last;
        }
        __syncthreads();
        if (*flag == 0u) return;
        if (wave < 4) {  // wave w takes row group w
          const float4 *qp = a.part + ((size_t)(r * 4 + wave) * Y + yc) * Z * MG * 64 + lane;
#pragma unroll
          for (int mg = 0; mg < MG; ++mg) {
            float4 v = load_coherent(qp + mg * 64);
            for (int z = 1; z < Z; ++z) {
              const float4 p = load_coherent(qp + ((size_t)z * MG + mg) * 64);
              v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
            }
            F[mg] = v;
          }
        }
      } else {
        // one workgroup per tile row: waves 0 .. 3 (split 0) hold row groups
        // 0 .. 3; every wave is done with the reduction buffer ys overlaps
        __syncthreads();
      }
      if (wave < 4) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          const float fv[4] = {F[mg].x, F[mg].y, F[mg].z, F[mg].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = mg * 16 + 4 * g + e;
            // the fused multiply-add with +0 rounds as the linear's sx * sum + 0
            if (t < xrows) ys[t * 64 + 16 * wave + i16] = fmaf(fv[e], sxv[mg][e], 0.0f);
          }
        }
      }
      if (tid < kXfWords) xtl[tid] = xtw;
      __syncthreads();
      // one token per wave at a time, lane l holding output l of the tile
      // row: Phi_s = D_L P H D_R (s >= 1), H (s = 0), the identity (s = -1)
      const XfTables &tl = *reinterpret_cast<const XfTables *>(xtl);
      const bool bad = useed < -1 || useed > kTransformSeeds;
      int src = lane;
      uint32_t fl = 0u, fr = 0u;
      if (useed >= 1 && !bad) {
        src = tl.perm[useed - 1][lane];
        fl = (uint32_t)(tl.dlm[useed - 1] >> lane) & 1u;
        fr = (uint32_t)(tl.drm[useed - 1] >> lane) & 1u;
      }
      for (int t = wave; t < xrows; t += WAVES) {
        float v = ys[t * 64 + lane];
        if (bad) {
          v = __builtin_nanf("");
        } else if (useed >= 0) {
          v = __uint_as_float(__float_as_uint(v) ^ (fr << 31));                          // D_R
          v = xf_fwht64(v, lane);                                                         // H
          v = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(v)));  // P: from perm[l]
          v = __uint_as_float(__float_as_uint(v) ^ (fl << 31));                          // D_L
        }
        if (a.bias) v += bv;
        a.Y[(size_t)(mbase + t) * a.N + (size_t)r * 64 + lane] = v;
      }
      return;
    }
    if (Z > 1) {
      // Chunked K: the workgroup's sum goes to slot zc of its row group; the
      // workgroup that completes the row block's set of Z (arrival counter,
      // reset by that workgroup) adds the slots in increasing zc, which
      // continues the increasing split order across workgroups.
      //   The slots are written and read with device-coherent accesses only
      // (agent-scope atomic stores and loads), so the hand-over needs no
      // cache-wide write-back or invalidation: each writing wave waits until
      // its stores have completed before the barrier that precedes the
      // counter increment, and the last workgroup reads the slots only after
      // its increment has returned.
      float4 *pp = a.part + ((size_t)(r * 4 + rg) * Y + yc) * Z * MG * 64 + lane;
      if (sp == 0) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) store_coherent(pp + ((size_t)zc * MG + mg) * 64, F[mg]);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      uint32_t *flag = reinterpret_cast<uint32_t *>(smem);  // LDS is free again
      if (tid == 0) {
        uint32_t *cp = a.cnt + (size_t)bx * Y + yc;
        const uint32_t prev = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t last = prev == (uint32_t)(Z - 1) ? 1u : 0u;
        if (last) __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
      }
      __syncthreads();
      if (*flag == 0u || sp != 0) return;
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        float4 v = load_coherent(pp + mg * 64);
        for (int z = 1; z < Z; ++z) {
          const float4 p = load_coherent(pp + ((size_t)z * MG + mg) * 64);
          v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        F[mg] = v;
      }
    } else if (sp != 0) {
      return;
    }
    const size_t n = (size_t)r * 64 + rg * 16 + i16;
    if (MODE == kValu) {
      const float b = a.bias ? a.bias[n] : 0.0f;
      if (g == 0) {
        const float fv[4] = {F[0].x, F[0].y, F[0].z, F[0].w};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (m < M) a.Y[(size_t)m * a.N + n] = GRP ? fv[m] + b : fv[m] * a.sx[m] + b;
      }
    } else {
      const float b = GRP ? (a.bias ? a.bias[n] : 0.0f) : bv;
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const float fv[4] = {F[mg].x, F[mg].y, F[mg].z, F[mg].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mbase + mg * 16 + 4 * g + e;
          if (m < M) a.Y[(size_t)m * a.N + n] = GRP ? fv[e] + b : fv[e] * sxv[mg][e] + b;
        }
      }
    }
  }
}

template <typename Kern, typename Args>
void launch_one(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const Args &args) {
  if (lds > 64 * 1024) (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, grid, block, lds, stream, args);
}

// Grid: row blocks (4R/RG) along x, token chunks along y, column chunks
// along z.
template <int BK, int MODE, int MG, int WAVES, int DEPTH, int XMODE, bool PARTIALS, bool INL, bool GRP,
          bool WNT, bool XF>
void launch_rg(const DecodePlan &p, int R, hipStream_t stream, const DArgs<INL, XF> &args) {
  const dim3 block(WAVES * 64);
  const dim3 grid(R * (4 / p.RG), args.ychunks, p.Z);
  switch (p.RG) {
    case 4: launch_one(decode_kernel<BK, MODE, MG, WAVES, 4, DEPTH, XMODE, PARTIALS, INL, GRP, WNT, XF>, grid, block, p.lds, stream, args); break;
    case 2: launch_one(decode_kernel<BK, MODE, MG, WAVES, 2, DEPTH, XMODE, PARTIALS, INL, GRP, WNT, XF>, grid, block, p.lds, stream, args); break;
    default: launch_one(decode_kernel<BK, MODE, MG, WAVES, 1, DEPTH, XMODE, PARTIALS, INL, GRP, WNT, XF>, grid, block, p.lds, stream, args); break;
  }
}

// Weights are loaded non-temporally when the call passes over them once
// (one token chunk): measured 4-10% faster where they stream from HBM.  A
// call of several token chunks re-reads them, and the later chunks find them
// in the last-level cache only if the first chunk's loads allocated there.
template <int BK, bool PARTIALS, bool INL, bool GRP, bool XF>
void launch_mode(const DecodePlan &p, int R, hipStream_t stream, const DArgs<INL, XF> &args) {
  if constexpr (!XF) {
    if (p.mode == kValu) {
      launch_rg<BK, kValu, 1, 16, kPrivDepth, kXPriv, PARTIALS, INL, GRP, true, XF>(p, R, stream, args);
      return;
    }
  }
  if (p.xmode == kXPriv) {
    if constexpr (BK == 128 && !XF) {
      if (p.depth == kPriv16Depth) {
        launch_rg<BK, kMfma, 1, 16, kPriv16Depth, kXPriv, PARTIALS, INL, GRP, true, XF>(p, R, stream, args);
        return;
      }
    }
    launch_rg<BK, kMfma, 1, 16, kPrivDepth, kXPriv, PARTIALS, INL, GRP, true, XF>(p, R, stream, args);
    return;
  }
  if constexpr (!PARTIALS && !GRP && !XF) {
    if (p.xmode == kXFused) {  // (6 tiles per batch: the FP32 rows' registers fit beside them)
      launch_rg<BK, kMfma, 1, 16, kSharedDepthN, kXFused, false, INL, false, true, false>(p, R, stream, args);
      return;
    }
  }
  // (the transformed route keeps the non-temporal loads for every call: one
  // set of kernels fewer to build)
  if (PARTIALS || XF || p.mchunks == 1) {
    switch (p.MG) {
      case 1: launch_rg<BK, kMfma, 1, 16, kSharedDepth1, kXShared, PARTIALS, INL, GRP, true, XF>(p, R, stream, args); break;
      case 2: launch_rg<BK, kMfma, 2, 16, kSharedDepthN, kXShared, PARTIALS, INL, GRP, true, XF>(p, R, stream, args); break;
      case 3: launch_rg<BK, kMfma, 3, 16, kSharedDepthW, kXShared, PARTIALS, INL, GRP, true, XF>(p, R, stream, args); break;
      default: launch_rg<BK, kMfma, 4, 16, kSharedDepthW, kXShared, PARTIALS, INL, GRP, true, XF>(p, R, stream, args); break;
    }
    return;
  }
  if constexpr (!PARTIALS && !XF) {
    switch (p.MG) {
      case 1: launch_rg<BK, kMfma, 1, 16, kSharedDepth1, kXShared, false, INL, GRP, false, XF>(p, R, stream, args); break;
      case 2: launch_rg<BK, kMfma, 2, 16, kSharedDepthN, kXShared, false, INL, GRP, false, XF>(p, R, stream, args); break;
      case 3: launch_rg<BK, kMfma, 3, 16, kSharedDepthW, kXShared, false, INL, GRP, false, XF>(p, R, stream, args); break;
      default: launch_rg<BK, kMfma, 4, 16, kSharedDepthW, kXShared, false, INL, GRP, false, XF>(p, R, stream, args); break;
    }
  }
}

// Whether a call passes the metadata inside the kernel arguments.
bool inline_meta(const PackedView &w, bool xform) {
  return w.meta && w.C <= 128 && kMetaStride * w.R <= (xform ? kInlineWordsXf : kInlineWords);
}

XfTables xf_tables(const TransformTables &t) {
  XfTables x{};
  for (int j = 0; j < kTransformSeeds; ++j)
    for (int e = 0; e < 64; ++e) {
      x.perm[j][e] = t.perm[j][e];
      if (t.dl[j][e] < 0) x.dlm[j] |= 1ull << e;
      if (t.dr[j][e] < 0) x.drm[j] |= 1ull << e;
    }
  return x;
}

// Scratch of the allocation-free decode entry point: the chunked-K
// workspace (arrival counters at the head, then the chunks' FP32 sums) in a
// file-scope device array, one copy per GPU, kept until the process ends.
// Host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (decode_scratch); the array's name is not a device
// address on the host.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *__restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_counters(void *ws, hipStream_t stream) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t *>(ws),
                     kDecodeCounters);
  return hipGetLastError();
}

hipError_t decode_scratch(hipStream_t stream, void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the arrival counters must start at zero; every decode call leaves them
    // zero.  A fill kernel, not a memset, so that a first call made under
    // stream capture records a kernel node.
    constexpr int words = kDecodeCounters;
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t *>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

namespace {

// The launches of one decode call (tables != nullptr: with the output
// transform in the epilogue; X != nullptr: the fused route from FP32
// activations, which the caller has checked with fused_ok).
hipError_t decode_launches(const PackedView &w, const int8_t *qx, const float *sx, int M,
                           const float *bias, float *Y, int split, void *ws, int32_t *P,
                           hipStream_t stream, bool grouped, const int8_t *useeds,
                           const TransformTables *tables, const float *X = nullptr) {
  const bool xf = tables != nullptr;
  DecodePlan p = X ? plan_decode_fused(w, M, split) : plan_decode(w, M, split, xf);
  if (!decode_plan_ok(p, w, xf) || p.ylaunch < 1) return hipErrorInvalidValue;
  if (grouped && M <= kValuMaxM) p.mode = kValu;
  DecodeArgs args;
  args.labels = w.labels; args.off4 = w.off4; args.off8 = w.off8;
  args.w4 = w.w4; args.w8 = w.w8; args.s4 = w.s4; args.s8 = w.s8;
  args.qx = qx; args.sx = sx; args.bias = bias;
  args.Y = Y; args.P = P;
  args.xf = X;
  args.N = w.N; args.K = w.K; args.R = w.R; args.C = w.C; args.T4 = w.T4; args.T8 = w.T8;
  args.M = M; args.label_words = (w.R * w.C + 31) / 32;
  args.Z = p.Z;
  args.kg64 = w.K / 64;
  args.xstride = p.xstride;
  args.cnt = nullptr;
  args.part = nullptr;
  if (p.ws_bytes > 0 && !P) {  // the products need no hand-over
    args.cnt = static_cast<uint32_t *>(ws);
    args.part = reinterpret_cast<float4 *>(static_cast<uint8_t *>(ws) + p.cnt_bytes);
  }
  XfArgs xa{};
  if (xf) {
    xa.useeds = useeds;
    xa.xt = xf_tables(*tables);
  }
  const bool inl = !P && !grouped && inline_meta(w, xf);
  // token ranges of ylaunch chunks of 16*MG tokens, one launch each
  const int mstep = p.ylaunch * 16 * p.MG;
  for (int m0 = 0; m0 < M; m0 += mstep) {
    DArgs<false, false> la;
    static_cast<DecodeArgs &>(la) = args;
    la.M = M - m0 < mstep ? M - m0 : mstep;
    if (qx) la.qx = qx + (size_t)m0 * w.K;
    // grouped scales: one row of K/64 per 16 tokens (launches start on a
    // multiple of 16 tokens; a single token is its own group)
    if (sx) la.sx = grouped ? sx + (size_t)(m0 / 16) * (w.K / 64) : sx + m0;
    if (Y) la.Y = Y + (size_t)m0 * w.N;
    if (P) la.P = P + (size_t)m0 * w.N * w.C;
    la.ychunks = p.mode == kValu || p.xmode != kXShared ? 1 : (la.M + 16 * p.MG - 1) / (16 * p.MG);
    if (P && grouped) {
      if (w.bK == 128) launch_mode<128, true, false, true>(p, w.R, stream, la);
      else launch_mode<64, true, false, true>(p, w.R, stream, la);
    } else if (P) {
      if (w.bK == 128) launch_mode<128, true, false, false>(p, w.R, stream, la);
      else launch_mode<64, true, false, false>(p, w.R, stream, la);
    } else if (grouped) {
      if (w.bK == 128) launch_mode<128, false, false, true>(p, w.R, stream, la);
      else launch_mode<64, false, false, true>(p, w.R, stream, la);
    } else if (xf && inl) {
      DArgs<true, true> li;
      static_cast<DecodeArgs &>(li) = la;
      li.xf = xa;
      std::memcpy(li.meta, w.meta, sizeof(uint32_t) * kMetaStride * w.R);
      if (w.bK == 128) launch_mode<128, false, true, false>(p, w.R, stream, li);
      else launch_mode<64, false, true, false>(p, w.R, stream, li);
    } else if (xf) {
      DArgs<false, true> lx;
      static_cast<DecodeArgs &>(lx) = la;
      lx.xf = xa;
      if (w.bK == 128) launch_mode<128, false, false, false>(p, w.R, stream, lx);
      else launch_mode<64, false, false, false>(p, w.R, stream, lx);
    } else if (inl) {
      DArgs<true, false> li;
      static_cast<DecodeArgs &>(li) = la;
      std::memcpy(li.meta, w.meta, sizeof(uint32_t) * kMetaStride * w.R);
      if (w.bK == 128) launch_mode<128, false, true, false>(p, w.R, stream, li);
      else launch_mode<64, false, true, false>(p, w.R, stream, li);
    } else {
      if (w.bK == 128) launch_mode<128, false, false, false>(p, w.R, stream, la);
      else launch_mode<64, false, false, false>(p, w.R, stream, la);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode(const PackedView &w, const int8_t *qx, const float *sx, int M,
                         const float *bias, float *Y, int split, void *ws, int32_t *P,
                         hipStream_t stream, bool grouped) {
  return decode_launches(w, qx, sx, M, bias, Y, split, ws, P, stream, grouped, nullptr, nullptr);
}

hipError_t launch_decode_transformed(const PackedView &w, const int8_t *qx, const float *sx, int M,
                                     const float *bias, float *Y, int split, void *ws,
                                     const int8_t *useeds, const TransformTables &t,
                                     hipStream_t stream) {
  return decode_launches(w, qx, sx, M, bias, Y, split, ws, nullptr, stream, false, useeds, &t);
}

hipError_t launch_decode_fp32(const PackedView &w, const float *X, int M, const float *bias, float *Y,
                              int split, void *ws, hipStream_t stream) {
  if (fused_ok(w, M, split))
    return decode_launches(w, nullptr, nullptr, M, bias, Y, split, nullptr, nullptr, stream, false,
                           nullptr, nullptr, X);
  // quantize into the workspace behind the decode workspace, then decode
  int8_t *qx = static_cast<int8_t *>(ws) + fp32_head_bytes(w, M, split);
  float *sx = reinterpret_cast<float *>(qx + (((size_t)M * w.K + 255) & ~(size_t)255));
  const hipError_t e = launch_quant_act(X, M, w.K, qx, sx, stream);
  if (e != hipSuccess) return e;
  return decode_launches(w, qx, sx, M, bias, Y, split, ws, nullptr, stream, false, nullptr, nullptr);
}

}  // namespace aq
