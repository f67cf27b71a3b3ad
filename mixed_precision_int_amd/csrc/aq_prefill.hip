// Compute-bound phase of the tile-aligned W4/W8 x A8 linear layer
// (AlignQuant Sec. 3.3 "Prefill weight reuse"; App. E.3, eq. 19).
//
// Workgroup = WM x WN wavefronts computing a (64 WM tokens) x (64 WN
// outputs) block: WN whole 64-row weight-tile rows, so within one
// input-tile column every wave multiplies exactly one weight tile and one
// precision.  Two workgroups share a CU; they are not synchronized with
// each other, so one's MFMAs overlap the other's VALU rescale.
//
// For each input-tile column j the block stages, double-buffered in LDS:
//   A: the BM x b_K INT8 activation slab, row-major with the 16-byte chunk
//      index XOR-swizzled by (row >> 1) so that the MFMA fragment reads are
//      free of bank conflicts;
//   B: the WN weight tiles widened to INT8 as 16-column panels
//      [panel][n][16] (the INT8 tile layout); INT4 tiles are widened x16 in
//      registers on the way in (see w4_lo16), which the rescale undoes with
//      an exact 1/16.
// Global loads of column j+1 are issued before the MFMAs of column j and
// written to the other LDS buffer after them.  Rows past M read row M-1
// (their outputs are never stored), so activation loads need no branch.
//
// Each wave runs v_mfma_i32_32x32x32_i8 on 2 x 2 fragments per 32 columns,
// then converts the INT32 tile product to FP32 and accumulates it with the
// tile's per-row weight scale (eq. 19); the token scale and the bias are
// applied once at the end.

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_tile_xform.h"

namespace aq {
namespace {

struct PrefillArgs {
  const uint8_t *labels;
  const int32_t *off4, *off8;
  const uint8_t *w4;
  const int8_t *w8;
  const float *s4, *s8;
  const int8_t *qx;
  const float *sx, *bias;
  float *Y;
  int32_t *P;
  int N, K, R, C, T4, T8, M, MB, NB, label_words;
  const int8_t *useeds;  // output transform (XFORM): per tile row seed (-1 .. 6)
  OutTables ot;
};

__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

template <int BK, int WM, int WN, bool PARTIALS, bool XFORM>
__global__ __launch_bounds__(64 * WM * WN, 8 / (WM * WN)) void prefill_kernel(const PrefillArgs a) {
  static_assert(!(PARTIALS && XFORM), "the debug products take no output transform");
  constexpr int NT = 64 * WM * WN;            // threads
  constexpr int BM = 64 * WM, BN = 64 * WN;   // block tile
  constexpr int NP = BK / 16;                 // 16-byte chunks per row of a tile column
  constexpr int KSTEPS = BK / 32;             // MFMA k-steps per tile column
  constexpr int A_CH = BM * NP / NT;          // activation chunks per thread
  constexpr int W8N = 64 * NP;                // 16-byte chunks of an INT8 tile
  constexpr int W4N = 32 * NP;                // 16-byte chunks of an INT4 tile
  constexpr int B8_CH = (W8N + NT - 1) / NT;  // INT8 chunks per thread per tile
  constexpr int B4_CH = (W4N + NT - 1) / NT;  // INT4 chunks per thread per tile
  static_assert(BM * NP % NT == 0, "activation slab must split evenly");

  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][NP * BN * 16];

  // Rasterization.  Hardware places block k on XCD k % 8, so logical block
  // L = (k % 8) * (G / 8) + k / 8 gives each XCD a contiguous range of L;
  // consecutive L then walk GROUP_M M-blocks down one N-block column before
  // moving right, so the blocks resident on an XCD at one time cover a
  // compact GROUP_M x (resident / GROUP_M) rectangle whose A and B
  // column slices are shared in that XCD's L2.
  constexpr int GROUP_M = 8;
  const int G = gridDim.x;
  const int kb = blockIdx.x;
  const int per = G / 8;
  const int L = (kb < per * 8) ? (kb % 8) * per + kb / 8 : kb;
  const int in_group = GROUP_M * a.NB;
  const int first_m = (L / in_group) * GROUP_M;
  const int gsize = min(a.MB - first_m, GROUP_M);
  const int bm = first_m + (L % in_group) % gsize;
  const int bn = (L % in_group) / gsize;
  const int m0 = bm * BM;
  const int r0 = WN * bn;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int rw = r0 + wn;  // this wave's weight-tile row
  const bool wave_live = rw < a.R;
  const int h = lane >> 5;

  // ---- per-thread activation chunk coordinates (fixed over j)
  // (byte offsets are 32-bit against a uniform base, so the address of every
  // load and LDS access is one scalar base plus a fixed per-lane offset)
  uint32_t a_src[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int it = 0; it < A_CH; ++it) {
    const int c = it * NT + tid;
    const int row = c / NP, p = c % NP;
    const int m = min(m0 + row, a.M - 1);
    a_src[it] = (uint32_t)m * (uint32_t)a.K + p * 16;
    a_dst[it] = row * BK + ((p ^ ((row >> 1) & (NP - 1))) * 16);
  }
  uint32_t b_src[B8_CH];
#pragma unroll
  for (int e = 0; e < B8_CH; ++e) b_src[e] = (uint32_t)(e * NT + tid) * 16u;
  // ---- per-lane fragment read offsets (fixed over j), for k-step u add 32u
  int af_off[2][KSTEPS], bf_off[2][KSTEPS];
#pragma unroll
  for (int u = 0; u < KSTEPS; ++u) {
    const int p = 2 * u + h;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int row = wm * 64 + f * 32 + (lane & 31);
      af_off[f][u] = row * BK + ((p ^ ((row >> 1) & (NP - 1))) * 16);
      const int n = wn * 64 + f * 32 + (lane & 31);
      bf_off[f][u] = (p * BN + n) * 16;
    }
  }

  // ---- eq. 16 walk of the WN tile rows (scalar)
  int nx4[WN], nx8[WN];
  uint64_t lbits[WN];
#pragma unroll
  for (int tt = 0; tt < WN; ++tt) {
    const int r = min(r0 + tt, a.R - 1);
    nx4[tt] = a.off4[r];
    nx8[tt] = a.off8[r];
    lbits[tt] = 0;
  }

  // ---- staging registers for the column being loaded
  v4i ra[A_CH];
  v4i rb[WN][B8_CH];
  int ld_is4[WN], ld_idx[WN];
  float ld_sc0 = 0.f, ld_sc1 = 0.f;

  // issue the global loads of tile column j.  Branch-free: every tile loads
  // B8_CH chunks per thread (an INT4 tile re-reads its own chunks past its
  // end), an absent or inconsistent tile re-reads tile 0 of a non-empty
  // buffer and is marked dead, and nothing loaded is used before the MFMAs of
  // the previous column have been issued.
#define AQ_LOAD_COLUMN(j)                                                                      \
  do {                                                                                         \
    const int j_ = (j);                                                                        \
    const int8_t *abase = a.qx + (size_t)j_ * BK;                                              \
    _Pragma("unroll") for (int it = 0; it < A_CH; ++it) ra[it] = ld16(abase + a_src[it]);     \
    _Pragma("unroll") for (int tt = 0; tt < WN; ++tt) {                                        \
      const int r = r0 + tt;                                                                   \
      if ((j_ & 63) == 0) lbits[tt] = label_bits64(a.labels, min(r, a.R - 1) * a.C + j_, a.label_words); \
      int l = (int)((lbits[tt] >> (j_ & 63)) & 1u);                                          \
      int id = l ? nx4[tt] : nx8[tt];                                                          \
      nx4[tt] += l;                                                                            \
      nx8[tt] += l ^ 1;                                                                        \
      const int ok = r < a.R && id >= 0 && id < (l ? a.T4 : a.T8);                             \
      if (!ok) { l = a.T4 > 0 ? 1 : 0; id = 0; }                                               \
      ld_is4[tt] = l;                                                                          \
      ld_idx[tt] = ok ? id : -1;                                                               \
      const uint8_t *src = l ? a.w4 + (size_t)id * (64 * BK / 2)                               \
                             : reinterpret_cast<const uint8_t *>(a.w8) + (size_t)id * (64 * BK); \
      /* an INT4 tile has half the chunks: chunk c >= W4N re-reads c mod W4N */                \
      const uint32_t wmask = l ? (uint32_t)W4N * 16u - 1u : (uint32_t)W8N * 16u - 1u;          \
      _Pragma("unroll") for (int e = 0; e < B8_CH; ++e) rb[tt][e] = ld16(src + (b_src[e] & wmask)); \
      if (tt == wn) {                                                                          \
        const float *sp = (l ? a.s4 : a.s8) + (size_t)id * 64 + (lane & 31);                  \
        ld_sc0 = sp[0];                                                                        \
        ld_sc1 = sp[32];                                                                       \
      }                                                                                        \
    }                                                                                          \
  } while (0)

  // write the staged column into LDS buffer st
#define AQ_STORE_COLUMN(st)                                                                    \
  do {                                                                                         \
    int8_t *As_ = As[(st)];                                                                    \
    int8_t *Bs_ = Bs[(st)];                                                                    \
    _Pragma("unroll") for (int it = 0; it < A_CH; ++it)                                        \
      *reinterpret_cast<v4i *>(As_ + a_dst[it]) = ra[it];                                      \
    _Pragma("unroll") for (int tt = 0; tt < WN; ++tt) {                                        \
      if (ld_idx[tt] < 0) continue;                                                            \
      if (ld_is4[tt]) {                                                                        \
        _Pragma("unroll") for (int e = 0; e < B4_CH; ++e) {                                    \
          const int c = e * NT + tid;                                                          \
          if (c < W4N) {                                                                       \
            const int q = c / 64, i = c % 64;                                                  \
            const v4i w = rb[tt][e];                                                           \
            *reinterpret_cast<v4i *>(Bs_ + ((2 * q) * BN + tt * 64 + i) * 16) =                \
                v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_lo16(w[2]), w4_lo16(w[3])};             \
            *reinterpret_cast<v4i *>(Bs_ + ((2 * q + 1) * BN + tt * 64 + i) * 16) =            \
                v4i{w4_hi16(w[0]), w4_hi16(w[1]), w4_hi16(w[2]), w4_hi16(w[3])};             \
          }                                                                                    \
        }                                                                                      \
      } else {                                                                                 \
        _Pragma("unroll") for (int e = 0; e < B8_CH; ++e) {                                    \
          const int c = e * NT + tid;                                                          \
          if (c < W8N) {                                                                       \
            const int p = c / 64, i = c % 64;                                                  \
            *reinterpret_cast<v4i *>(Bs_ + (p * BN + tt * 64 + i) * 16) = rb[tt][e];           \
          }                                                                                    \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
  } while (0)

  float F[2][2][16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][fn][e] = 0.f;

  AQ_LOAD_COLUMN(0);
  AQ_STORE_COLUMN(0);
  int cur_is4 = ld_is4[wn], cur_idx = wave_live ? ld_idx[wn] : -1;
  float cur_sc0 = ld_is4[wn] ? ld_sc0 * 0.0625f : ld_sc0;
  float cur_sc1 = ld_is4[wn] ? ld_sc1 * 0.0625f : ld_sc1;
  __syncthreads();

#define AQ_COLUMN_BODY(jarg, ST_) \
    const int jc_ = (jarg); \
    const bool more = jc_ + 1 < a.C; \
    if (more) AQ_LOAD_COLUMN(jc_ + 1); \
 \
    if (cur_idx >= 0) { \
      const int8_t *As_ = As[ST_]; \
      const int8_t *Bs_ = Bs[ST_]; \
      v16i acc[2][2]; \
_Pragma("unroll") \
      for (int fm = 0; fm < 2; ++fm) \
_Pragma("unroll") \
        for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = v16i{0}; \
_Pragma("unroll") \
      for (int u = 0; u < KSTEPS; ++u) { \
        const v4i a0 = *reinterpret_cast<const v4i *>(As_ + af_off[0][u]); \
        const v4i a1 = *reinterpret_cast<const v4i *>(As_ + af_off[1][u]); \
        const v4i b0 = *reinterpret_cast<const v4i *>(Bs_ + bf_off[0][u]); \
        const v4i b1 = *reinterpret_cast<const v4i *>(Bs_ + bf_off[1][u]); \
        acc[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, acc[0][0], 0, 0, 0); \
        acc[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b1, acc[0][1], 0, 0, 0); \
        acc[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, acc[1][0], 0, 0, 0); \
        acc[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, acc[1][1], 0, 0, 0); \
      } \
      if constexpr (PARTIALS) { \
        /* 32x32 MFMA result: column (output n) = lane & 31, */ \
        /* row (token) = 8 (e / 4) + 4 (lane >> 5) + (e & 3). */ \
_Pragma("unroll") \
        for (int fm = 0; fm < 2; ++fm) \
_Pragma("unroll") \
          for (int fn = 0; fn < 2; ++fn) \
_Pragma("unroll") \
            for (int e = 0; e < 16; ++e) { \
              const int m = m0 + wm * 64 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3); \
              const size_t n = (size_t)rw * 64 + fn * 32 + (lane & 31); \
              if (m < a.M) { \
                const int v = acc[fm][fn][e]; \
                a.P[((size_t)m * a.N + n) * a.C + jc_] = cur_is4 ? (v >> 4) : v; \
              } \
            } \
      } else { \
_Pragma("unroll") \
        for (int fm = 0; fm < 2; ++fm) \
_Pragma("unroll") \
          for (int e = 0; e < 16; ++e) { \
            F[fm][0][e] = fmaf((float)acc[fm][0][e], cur_sc0, F[fm][0][e]); \
            F[fm][1][e] = fmaf((float)acc[fm][1][e], cur_sc1, F[fm][1][e]); \
          } \
      } \
    } \
 \
    if (more) { \
      AQ_STORE_COLUMN(ST_ ^ 1); \
      cur_is4 = ld_is4[wn]; \
      cur_idx = wave_live ? ld_idx[wn] : -1; \
      cur_sc0 = ld_is4[wn] ? ld_sc0 * 0.0625f : ld_sc0; \
      cur_sc1 = ld_is4[wn] ? ld_sc1 * 0.0625f : ld_sc1; \
    } \
    __syncthreads();

  for (int j = 0; j < a.C; j += 2) {
    {
      AQ_COLUMN_BODY(j, 0)
    }
    if (j + 1 < a.C) {
      AQ_COLUMN_BODY(j + 1, 1)
    }
  }
#undef AQ_COLUMN_BODY
#undef AQ_LOAD_COLUMN
#undef AQ_STORE_COLUMN

  if constexpr (!PARTIALS) {
    if (!wave_live) return;
    // XFORM: Y = Y~ U on this wave's tile row (a token's 64 outputs sit in
    // one half-wave), before the token scale and the bias
    if constexpr (XFORM) out_transform<2>(F, a.useeds[rw], lane, a.ot);
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3);
        if (m >= a.M) continue;
        const float sxm = a.sx[m];
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          const size_t n = (size_t)rw * 64 + fn * 32 + (lane & 31);
          float v = F[fm][fn][e] * sxm;
          if (a.bias) v += a.bias[n];
          a.Y[(size_t)m * a.N + n] = v;
        }
      }
  }
}

template <int BK, int WM, int WN>
void launch_cfg(bool partials, hipStream_t stream, const PrefillArgs &args) {
  const dim3 grid(args.MB * args.NB);
  const dim3 block(64 * WM * WN);
  if (partials)
    hipLaunchKernelGGL((prefill_kernel<BK, WM, WN, true, false>), grid, block, 0, stream, args);
  else if (args.useeds)
    hipLaunchKernelGGL((prefill_kernel<BK, WM, WN, false, true>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((prefill_kernel<BK, WM, WN, false, false>), grid, block, 0, stream, args);
}

}  // namespace

hipError_t launch_prefill(const PackedView &w, const int8_t *qx, const float *sx, int M,
                          const float *bias, float *Y, int32_t *P, hipStream_t stream,
                          const int8_t *useeds, const aq_transform_tables *tables) {
  constexpr int WM = 2, WN = 2;
  PrefillArgs args;
  args.useeds = useeds && tables && !P ? useeds : nullptr;
  args.ot = args.useeds ? out_tables(*tables) : OutTables{};
  args.labels = w.labels; args.off4 = w.off4; args.off8 = w.off8;
  args.w4 = w.w4; args.w8 = w.w8; args.s4 = w.s4; args.s8 = w.s8;
  args.qx = qx; args.sx = sx; args.bias = bias; args.Y = Y; args.P = P;
  args.N = w.N; args.K = w.K; args.R = w.R; args.C = w.C; args.T4 = w.T4; args.T8 = w.T8;
  args.M = M;
  args.label_words = (w.R * w.C + 31) / 32;
  args.MB = (M + 64 * WM - 1) / (64 * WM);
  args.NB = (w.R + WN - 1) / WN;
  if (w.bK == 128) launch_cfg<128, WM, WN>(P != nullptr, stream, args);
  else launch_cfg<64, WM, WN>(P != nullptr, stream, args);
  return hipGetLastError();
}

}  // namespace aq
