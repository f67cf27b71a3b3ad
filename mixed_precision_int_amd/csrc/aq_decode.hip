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
//            memory instead.
//
// Products (the pages split decode the same way, Table 5):
//   M = 1 : v_dot4_i32_i8 on the vector ALU (a 4-way byte dot product); a
//           lane accumulates its 32 columns per tile and the four k-groups
//           are summed across lanes (swizzle / permute) before the split
//           reduction;
//   M > 1 : v_mfma_i32_16x16x64_i8 with up to 16 tokens as the A operand and
//           the 16 weight rows as the B operand, C[token 4g+e][row i16]; per
//           extra token the byte dot products would cost the vector ALU and
//           LDS a full operand pass each.
// Each tile's INT32 product is rescaled by its per-row FP32 scale into FP32
// accumulators (eq. 19).  INT4 tiles are widened x16 (see w4_lo16), so their
// scale is multiplied by the exact factor 1/16.

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

constexpr int kLdsBudget = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kValuMaxM = 1;            // largest M on the vector-ALU path
constexpr int kPrivMaxM = 4;            // largest M with per-wave activation slices
constexpr int kPrivDepth = 8;           // tiles per batch with per-wave activation slices
enum { kValu = 0, kMfma = 1 };
// Where the MFMA/VALU activation operands come from: a per-wave LDS slice
// of the batch, the workgroup's LDS copy of its tokens, or global memory.
enum { kXPriv = 0, kXShared = 1, kXGlobal = 2 };

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
  int N, K, R, C, T4, T8, M, label_words;
};

__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }
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
template <int BK>
__device__ __forceinline__ v4i x_operand(const int8_t *row, int colbase, int g, int u, int is4, int sw) {
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

template <int BK, int MODE, int MG, int WAVES, int RG, int DEPTH, int XMODE, bool PARTIALS>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(const DecodeArgs a) {
  constexpr int KS = BK / 64;    // MFMA steps (16-byte operands per lane) per tile
  constexpr int S = WAVES / RG;  // splits per row group
  constexpr int NT = WAVES * 64;
  constexpr int XU = 8;          // activation granules per thread per staging pass
  constexpr int XW = DEPTH * BK; // bytes of one token's activations per batch (per-wave slices)
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blocks_per_row = 4 / RG;
  const int r = blockIdx.x / blocks_per_row;
  const int rgl = wave % RG;  // row group inside the block
  const int rg = (blockIdx.x % blocks_per_row) * RG + rgl;
  const int sp = wave / RG;   // split of this wave
  const int C = a.C, K = a.K, M = a.M;
  const int c0 = (C * sp) / S;
  const int c1 = (C * (sp + 1)) / S;
  const int mbase = blockIdx.y * 16 * MG;
  const int xrows = MODE == kValu ? M : min(M - mbase, 16 * MG);  // token rows of this block
  const int g = lane >> 4, i16 = lane & 15;
  const int rowoff = rg * 256 + i16 * 16;  // this lane's row inside a 1 KB panel
  const uint8_t *__restrict__ w4p = a.w4;
  const uint8_t *__restrict__ w8p = reinterpret_cast<const uint8_t *>(a.w8);
  const int T4 = a.T4, T8 = a.T8;
  const int kg = K >> 4;                      // 16-byte granules per activation row
  const int xmask = (kg & 15) == 0 ? 15 : 0;  // granule swizzle (stays inside the row)
  // LDS: per-wave slices [WAVES][M][DEPTH*BK], or the block's [16*MG][K]
  // activations (granules swizzled by row); then the split reduction buffer
  // [WAVES][MG][64] float4.
  int8_t *xs = reinterpret_cast<int8_t *>(smem);
  int8_t *xw = xs + wave * M * XW;
  const int xbytes = XMODE == kXPriv ? WAVES * M * XW : XMODE == kXShared ? ((16 * MG * K + 15) & ~15) : 0;
  float4 *red = reinterpret_cast<float4 *>(smem + xbytes);

  // ---- MFMA path: block activation staging loads (independent of the
  // metadata), issued first
  v4i xb[XU];
  const int8_t *xsrc = a.qx + (size_t)mbase * K;
  const bool xstage = XMODE == kXShared;
  const int xgran = xstage ? xrows * kg : 0;
  if (xstage) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      if (u * NT < xgran) {  // uniform: only the passes the block needs
        const int q = min(tid + u * NT, xgran - 1);
        xb[u] = load16(xsrc + (size_t)q * 16);
      }
    }
  }

  // ---- eq. 16 bookkeeping: the row's offsets and label words in one batch
  // of scalar loads.  The label window below depends on the offsets (a
  // guard that valid metadata never trips), so the compiler cannot defer the
  // offset loads to their later use: all seven share one wait.
  const int tb = r * C;
  const bool fastlab = C <= 128;
  const int o4 = a.off4[r], o8 = a.off8[r];
  uint32_t lw[5];
  {
    const uint32_t *wd = reinterpret_cast<const uint32_t *>(a.labels);
    const int w0 = tb >> 5, last = a.label_words - 1;
#pragma unroll
    for (int k = 0; k < 5; ++k) lw[k] = wd[min(w0 + k, last)];
  }
  if ((o4 | o8) < 0) lw[4] = 0u;  // negative row offsets: inconsistent metadata
  uint64_t wlo, whi;
  label_window(lw, tb, wlo, whi);
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
  v4i xv[kPrivMaxM];  // per-wave slices: this lane's granule of the batch, per token

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
          if (BK == 128) {                                                                      \
            if (is4) {                                                                          \
              W[d][0] = load16(w4p + (size_t)idx * 4096 + g * 1024 + rowoff);                   \
            } else {                                                                            \
              const uint8_t *base = w8p + (size_t)idx * 8192 + (2 * g) * 1024 + rowoff;         \
              W[d][0] = load16(base);                                                           \
              W[d][1] = load16(base + 1024);                                                    \
            }                                                                                   \
          } else {                                                                              \
            if (is4) {                                                                          \
              const uint2 lo = load8(w4p + (size_t)idx * 2048 + (g >> 1) * 1024 + rowoff + 8 * (g & 1)); \
              W[d][0] = v4i{(int)lo.x, (int)lo.y, 0, 0};                                        \
            } else {                                                                            \
              W[d][0] = load16(w8p + (size_t)idx * 4096 + g * 1024 + rowoff);                   \
            }                                                                                   \
          }                                                                                     \
          SC[d] = (is4 ? a.s4 : a.s8)[(size_t)idx * 64 + rg * 16 + i16];                        \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
    if (XMODE == kXPriv) {                                                                      \
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
        *reinterpret_cast<v4i *>(xs + row * K + 16 * (cg ^ (row & xmask))) = xb[u];
      }
    }
    for (int q0 = XU * NT; q0 < xgran; q0 += XU * NT) {  // large blocks only
      v4i xt[XU];
#pragma unroll
      for (int u = 0; u < XU; ++u) xt[u] = load16(xsrc + (size_t)min(q0 + tid + u * NT, xgran - 1) * 16);
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int q = q0 + tid + u * NT;
        if (q < xgran) {
          const int row = q / kg, cg = q - row * kg;
          *reinterpret_cast<v4i *>(xs + row * K + 16 * (cg ^ (row & xmask))) = xt[u];
        }
      }
    }
  }
  AQ_DECODE_ISSUE(c0);
  if (xstage) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS writes done; vmcnt left open
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  for (int t0 = c0; t0 < c1; t0 += DEPTH) {
    if (t0 != c0) AQ_DECODE_ISSUE(t0);
    if (XMODE == kXPriv) {  // the wave's own activation slice; read back by this wave only
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
      if (BK == 128) {
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
          const int8_t *xr = XMODE == kXPriv ? xw + trow * XW
                           : XMODE == kXShared ? xs + trow * K : xsrc + (size_t)trow * K;
          const int xcol = XMODE == kXPriv ? d * BK : jt * BK;
          const int sw = XMODE == kXShared ? (trow & xmask) : 0;
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const v4i xop = x_operand<BK>(xr, xcol, g, u, is4, sw);
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
      } else {
        // vector ALU: the one token, this lane's 16*KS columns
        int acc[kValuMaxM];
#pragma unroll
        for (int m = 0; m < kValuMaxM; ++m) {
          acc[m] = 0;
          if (m < M) {
#pragma unroll
            for (int u = 0; u < KS; ++u) {
              const v4i xop = x_operand<BK>(xw + m * XW, d * BK, g, u, is4, 0);
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
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) red[(wave * MG + mg) * 64 + lane] = F[mg];
      __syncthreads();
      if (sp != 0) return;
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
    const size_t n = (size_t)r * 64 + rg * 16 + i16;
    const float b = a.bias ? a.bias[n] : 0.0f;
    if (MODE == kValu) {
      if (g == 0) {
        const float fv[4] = {F[0].x, F[0].y, F[0].z, F[0].w};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (m < M) a.Y[(size_t)m * a.N + n] = fv[m] * a.sx[m] + b;
      }
    } else {
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const float fv[4] = {F[mg].x, F[mg].y, F[mg].z, F[mg].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mbase + mg * 16 + 4 * g + e;
          if (m < M) a.Y[(size_t)m * a.N + n] = fv[e] * a.sx[m] + b;
        }
      }
    }
  }
}

template <typename Kern>
void launch_one(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const DecodeArgs &args) {
  if (lds > 64 * 1024) (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, grid, block, lds, stream, args);
}

template <int BK, int MODE, int MG, int WAVES, int DEPTH, int XMODE, bool PARTIALS>
void launch_rg(int RG, int R, int mchunks, size_t lds, hipStream_t stream, const DecodeArgs &args) {
  const dim3 block(WAVES * 64);
  switch (RG) {
    case 4: launch_one(decode_kernel<BK, MODE, MG, WAVES, 4, DEPTH, XMODE, PARTIALS>, dim3(R, mchunks), block, lds, stream, args); break;
    case 2: launch_one(decode_kernel<BK, MODE, MG, WAVES, 2, DEPTH, XMODE, PARTIALS>, dim3(R * 2, mchunks), block, lds, stream, args); break;
    default: launch_one(decode_kernel<BK, MODE, MG, WAVES, 1, DEPTH, XMODE, PARTIALS>, dim3(R * 4, mchunks), block, lds, stream, args); break;
  }
}

template <int BK, bool PARTIALS>
void launch_mode(int mode, int xmode, int MG, int RG, int R, int mchunks, size_t lds, hipStream_t stream,
                 const DecodeArgs &args) {
  if (mode == kValu) {
    launch_rg<BK, kValu, 1, 16, kPrivDepth, kXPriv, PARTIALS>(RG, R, 1, lds, stream, args);
    return;
  }
  if (xmode == kXPriv) {
    launch_rg<BK, kMfma, 1, 16, kPrivDepth, kXPriv, PARTIALS>(RG, R, 1, lds, stream, args);
    return;
  }
  if (xmode == kXShared) {
    switch (MG) {
      case 1: launch_rg<BK, kMfma, 1, 16, 8, kXShared, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
      case 2: launch_rg<BK, kMfma, 2, 16, 6, kXShared, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
      case 3: launch_rg<BK, kMfma, 3, 8, 6, kXShared, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
      default: launch_rg<BK, kMfma, 4, 8, 6, kXShared, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    }
    return;
  }
  switch (MG) {
    case 1: launch_rg<BK, kMfma, 1, 16, 8, kXGlobal, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    case 2: launch_rg<BK, kMfma, 2, 16, 6, kXGlobal, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    case 3: launch_rg<BK, kMfma, 3, 8, 6, kXGlobal, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    default: launch_rg<BK, kMfma, 4, 8, 6, kXGlobal, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
  }
}

}  // namespace

int decode_mgroups(int M) { return M >= 49 ? 4 : (M + 15) / 16; }

int decode_mchunks(int M) {
  const int MG = decode_mgroups(M);
  return (M + 16 * MG - 1) / (16 * MG);
}

int decode_waves(int M) { return decode_mgroups(M) <= 2 ? 16 : 8; }

// Row groups per workgroup: the fewest that still let the whole grid
// (4R/RG workgroups, one per CU at this occupancy) run in a single round on
// the 256 CUs; more row groups per workgroup means fewer, longer splits.
int decode_rowgroups(const PackedView &w, int M) {
  (void)M;
  const int cus = 256;
  if (4 * w.R <= cus) return 1;
  if (2 * w.R <= cus) return 2;
  return 4;
}

int decode_split(const PackedView &w, int M) {
  return decode_waves(M) / decode_rowgroups(w, M);
}

bool decode_split_supported(int M, int S) {
  const int W = decode_waves(M);
  return S == W || S == W / 2 || S == W / 4;
}

size_t decode_workspace_bytes(const PackedView &, int, int) { return 0; }

hipError_t launch_decode(const PackedView &w, const int8_t *qx, const float *sx, int M,
                         const float *bias, float *Y, int S, void *ws, int32_t *P,
                         hipStream_t stream) {
  (void)ws;
  DecodeArgs args;
  args.labels = w.labels; args.off4 = w.off4; args.off8 = w.off8;
  args.w4 = w.w4; args.w8 = w.w8; args.s4 = w.s4; args.s8 = w.s8;
  args.qx = qx; args.sx = sx; args.bias = bias;
  args.Y = Y; args.P = P;
  args.N = w.N; args.K = w.K; args.R = w.R; args.C = w.C; args.T4 = w.T4; args.T8 = w.T8;
  args.M = M; args.label_words = (w.R * w.C + 31) / 32;
  const int MG = decode_mgroups(M);
  const int waves = decode_waves(M);
  // split S (waves per row group) selects the row groups per workgroup
  int RG = S > 0 ? waves / S : decode_rowgroups(w, M);
  if (RG != 1 && RG != 2 && RG != 4) RG = decode_rowgroups(w, M);
  const int mchunks = decode_mchunks(M);
  // Products: vector ALU for one token, MFMA otherwise.  Activations: a
  // per-wave LDS slice of each batch for M <= 4 (no workgroup barrier),
  // else the block's [16*MG][K] tokens in LDS when they fit, else global.
  const size_t red = (size_t)waves * MG * 64 * sizeof(float4);
  const int mode = M <= kValuMaxM ? kValu : kMfma;
  int xmode;
  size_t xbytes;
  if (M <= kPrivMaxM) {
    xmode = kXPriv;
    xbytes = (size_t)waves * M * kPrivDepth * w.bK;
  } else {
    xbytes = ((size_t)16 * MG * w.K + 15) & ~(size_t)15;
    xmode = xbytes + red <= (size_t)kLdsBudget ? kXShared : kXGlobal;
    if (xmode == kXGlobal) xbytes = 0;
  }
  const size_t lds = xbytes + red;
  if (w.bK == 128) {
    if (P) launch_mode<128, true>(mode, xmode, MG, RG, w.R, mchunks, lds, stream, args);
    else launch_mode<128, false>(mode, xmode, MG, RG, w.R, mchunks, lds, stream, args);
  } else {
    if (P) launch_mode<64, true>(mode, xmode, MG, RG, w.R, mchunks, lds, stream, args);
    else launch_mode<64, false>(mode, xmode, MG, RG, w.R, mchunks, lds, stream, args);
  }
  return hipGetLastError();
}

}  // namespace aq
