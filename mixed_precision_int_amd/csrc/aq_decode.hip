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
// The INT8 activations of the workgroup's tokens are staged once in LDS
// (coalesced 16-byte loads issued together with the metadata loads;
// 16-byte granules XOR-swizzled by token row so that the 16 rows one MFMA
// operand reads fall in distinct banks); the workgroup barrier that
// publishes them is taken while the first weight batch is in flight.  When
// they do not fit, lanes read them from global memory instead.
//
// Products:
//   M <= 4  : v_dot4_i32_i8 on the vector ALU (the pages' one-token decode
//             uses a 4-way byte dot product, Table 5); a lane accumulates its
//             32 columns per tile and the four k-groups are summed across
//             lanes (swizzle / permute) before the split reduction.
//   M  > 4  : v_mfma_i32_16x16x64_i8 with up to 16 tokens as the A operand and
//             the 16 weight rows as the B operand, C[token 4g+e][row i16]; at
//             these token counts the byte dot products would outrun the
//             vector ALU before HBM.
// Each tile's INT32 product is rescaled by its per-row FP32 scale into FP32
// accumulators (eq. 19).  INT4 tiles are widened x16 (see w4_lo16), so their
// scale is multiplied by the exact factor 1/16.

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

constexpr int kLdsBudget = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kValuMaxM = 4;            // largest M on the vector-ALU path
enum { kValu = 0, kMfma = 1 };

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

template <int BK, int MODE, int MG, int WAVES, int RG, int DEPTH, bool XLDS, bool PARTIALS>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(const DecodeArgs a) {
  constexpr int KS = BK / 64;    // MFMA steps (16-byte operands per lane) per tile
  constexpr int S = WAVES / RG;  // splits per row group
  constexpr int NT = WAVES * 64;
  constexpr int XU = 8;          // activation granules per thread per staging pass
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
  const int kg = K >> 4;                        // 16-byte granules per activation row
  const int xmask = (kg & 15) == 0 ? 15 : 0;    // granule swizzle (stays inside the row)
  int8_t *xs = reinterpret_cast<int8_t *>(smem);  // [xrows][K], granules swizzled
  const int xbytes = ((MODE == kValu ? M : 16 * MG) * K + 15) & ~15;
  float4 *red = reinterpret_cast<float4 *>(smem + (XLDS ? xbytes : 0));  // [WAVES][MG][64]

  // ---- activation staging loads (independent of the metadata), issued first
  v4i xb[XU];
  const int8_t *xsrc = a.qx + (size_t)mbase * K;
  const int xgran = XLDS ? xrows * kg : 0;
  if (XLDS) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      if (u * NT < xgran) {  // uniform: only the passes the block needs
        const int q = min(tid + u * NT, xgran - 1);
        xb[u] = load16(xsrc + (size_t)q * 16);
      }
    }
  }

  // ---- eq. 16 bookkeeping: the row's offsets and label words in one batch
  // of scalar loads, all issued before the single wait (the empty asm
  // consumes them, so none is sunk past the others' use).
  const int tb = r * C;
  const bool fastlab = C <= 128;
  int o4 = a.off4[r], o8 = a.off8[r];
  uint32_t lw[5];
  {
    const uint32_t *wd = reinterpret_cast<const uint32_t *>(a.labels);
    const int w0 = tb >> 5, last = a.label_words - 1;
#pragma unroll
    for (int k = 0; k < 5; ++k) lw[k] = wd[min(w0 + k, last)];
  }
  asm volatile("" : "+s"(o4), "+s"(o8), "+s"(lw[0]), "+s"(lw[1]), "+s"(lw[2]), "+s"(lw[3]), "+s"(lw[4]));
  uint64_t wlo, whi;
  label_window(lw, tb, wlo, whi);
  int n4;
  if (fastlab) {
    n4 = c0 <= 64 ? __popcll(wlo & low_mask(c0))
                  : __popcll(wlo) + __popcll(whi & low_mask(c0 - 64));
  } else {
    n4 = count_int4(a.labels, tb, c0, a.label_words);
  }
  int idx4 = o4 + n4;
  int idx8 = o8 + (c0 - n4);

  // Activation rows of this lane (global fallback; padding tokens read the
  // last real row, their outputs are never stored).
  float4 F[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) F[mg] = make_float4(0.f, 0.f, 0.f, 0.f);

  v4i W[DEPTH][2];
  float SC[DEPTH];
  int live[DEPTH], is4v[DEPTH], jv[DEPTH];

  // Issue the loads of the live tiles among t0 .. t0+DEPTH-1 of the split:
  // the rows' 16-byte panel chunks (two for an INT8 tile at b_K = 128, one
  // otherwise) and the lane's row scale.  Live tiles are a prefix; the
  // branches are uniform.
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
  }

  // ---- activations into LDS (their loads were issued with the metadata
  // batch), then the first weight batch, then one barrier while it is in
  // flight
  if (XLDS) {
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
  if (XLDS) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS writes done; vmcnt left open
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Activation operand of token row t (relative to mbase) at global column
  // col (16 bytes; for b_K = 64 INT4 two 8-byte halves at col and col + 16).
#define AQ_XROW_PTR_G(t_) (a.qx + (size_t)(mbase + (t_)) * K)

  for (int t0 = c0; t0 < c1; t0 += DEPTH) {
    if (t0 != c0) AQ_DECODE_ISSUE(t0);
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
      // column of step u's 16 bytes (b_K = 64 INT4: first 8-byte half)
      const int colbase = jt * BK;
#define AQ_XCOL(u_) (BK == 128 ? colbase + 32 * g + 16 * (u_)                                  \
                               : (is4 ? colbase + 32 * (g >> 1) + 8 * (g & 1) : colbase + 16 * g))
#define AQ_XLOAD(dst_, trow_, u_)                                                               \
  {                                                                                             \
    const int trw = (trow_);                                                                    \
    const int col = AQ_XCOL(u_);                                                                \
    if (XLDS) {                                                                                 \
      const int8_t *xr = xs + trw * K;                                                          \
      const int sw = trw & xmask;                                                               \
      if (BK == 64 && is4) {                                                                    \
        const int cga = col >> 4, cgb = (col + 16) >> 4, in = col & 15;                         \
        const uint2 p0 = *reinterpret_cast<const uint2 *>(xr + 16 * (cga ^ sw) + in);          \
        const uint2 p1 = *reinterpret_cast<const uint2 *>(xr + 16 * (cgb ^ sw) + in);          \
        dst_ = v4i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y};                                 \
      } else {                                                                                  \
        dst_ = *reinterpret_cast<const v4i *>(xr + 16 * ((col >> 4) ^ sw));                    \
      }                                                                                         \
    } else {                                                                                    \
      const int8_t *xr = AQ_XROW_PTR_G(trw);                                                    \
      if (BK == 64 && is4) {                                                                    \
        const uint2 p0 = load8(xr + col), p1 = load8(xr + col + 16);                            \
        dst_ = v4i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y};                                 \
      } else {                                                                                  \
        dst_ = load16(xr + col);                                                                \
      }                                                                                         \
    }                                                                                           \
  }
      if (MODE == kMfma) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          const int trow = min(mg * 16 + i16, xrows - 1);
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            v4i xop;
            AQ_XLOAD(xop, trow, u);
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
        // vector ALU: tokens 0 .. min(M, 4)-1, each lane its 16*KS*... columns
        int acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[m] = 0;
          if (m < M) {
#pragma unroll
            for (int u = 0; u < KS; ++u) {
              v4i xop;
              AQ_XLOAD(xop, m, u);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[m] = __builtin_amdgcn_sdot4(wop[u][e], xop[e], acc[m], false);
            }
          }
        }
        if constexpr (PARTIALS) {
          const size_t n = (size_t)r * 64 + rg * 16 + i16;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if (m < M) {
              const int v = sum_kgroups_i(acc[m]);
              if (g == 0) a.P[((size_t)m * a.N + n) * C + jt] = is4 ? (v >> 4) : v;
            }
          }
        } else {
          F[0].x = fmaf((float)acc[0], sc, F[0].x);
          F[0].y = fmaf((float)acc[1], sc, F[0].y);
          F[0].z = fmaf((float)acc[2], sc, F[0].z);
          F[0].w = fmaf((float)acc[3], sc, F[0].w);
        }
      }
#undef AQ_XLOAD
#undef AQ_XCOL
    }
  }
#undef AQ_DECODE_ISSUE
#undef AQ_XROW_PTR_G

  if constexpr (!PARTIALS) {
    if (MODE == kValu) {  // sum the four k-groups of each row
      F[0].x = sum_kgroups(F[0].x);
      F[0].y = sum_kgroups(F[0].y);
      F[0].z = sum_kgroups(F[0].z);
      F[0].w = sum_kgroups(F[0].w);
    }
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

template <int BK, int MODE, int MG, int WAVES, int DEPTH, bool XLDS, bool PARTIALS>
void launch_rg(int RG, int R, int mchunks, size_t lds, hipStream_t stream, const DecodeArgs &args) {
  const dim3 block(WAVES * 64);
  switch (RG) {
    case 4: launch_one(decode_kernel<BK, MODE, MG, WAVES, 4, DEPTH, XLDS, PARTIALS>, dim3(R, mchunks), block, lds, stream, args); break;
    case 2: launch_one(decode_kernel<BK, MODE, MG, WAVES, 2, DEPTH, XLDS, PARTIALS>, dim3(R * 2, mchunks), block, lds, stream, args); break;
    default: launch_one(decode_kernel<BK, MODE, MG, WAVES, 1, DEPTH, XLDS, PARTIALS>, dim3(R * 4, mchunks), block, lds, stream, args); break;
  }
}

template <int BK, bool XLDS, bool PARTIALS>
void launch_mg(int mode, int MG, int RG, int R, int mchunks, size_t lds, hipStream_t stream,
               const DecodeArgs &args) {
  if (mode == kValu) {
    launch_rg<BK, kValu, 1, 16, 8, true, PARTIALS>(RG, R, 1, lds, stream, args);
    return;
  }
  switch (MG) {
    case 1: launch_rg<BK, kMfma, 1, 16, 8, XLDS, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    case 2: launch_rg<BK, kMfma, 2, 16, 6, XLDS, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    case 3: launch_rg<BK, kMfma, 3, 8, 6, XLDS, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
    default: launch_rg<BK, kMfma, 4, 8, 6, XLDS, PARTIALS>(RG, R, mchunks, lds, stream, args); break;
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
  // LDS: staged activations (when they fit) + split-reduction buffer
  const size_t red = (size_t)waves * MG * 64 * sizeof(float4);
  int mode = M <= kValuMaxM ? kValu : kMfma;
  const size_t xrows = mode == kValu ? (size_t)M : (size_t)16 * MG;
  const size_t xbytes = (xrows * (size_t)w.K + 15) & ~(size_t)15;
  const bool xlds = xbytes + red <= (size_t)kLdsBudget;
  if (mode == kValu && !xlds) mode = kMfma;  // very long rows: global activation reads
  const size_t lds = (mode == kValu || xlds) ? xbytes + red : red;
  if (P) {
    if (w.bK == 128) {
      if (xlds) launch_mg<128, true, true>(mode, MG, RG, w.R, mchunks, lds, stream, args);
      else launch_mg<128, false, true>(mode, MG, RG, w.R, mchunks, lds, stream, args);
    } else {
      if (xlds) launch_mg<64, true, true>(mode, MG, RG, w.R, mchunks, lds, stream, args);
      else launch_mg<64, false, true>(mode, MG, RG, w.R, mchunks, lds, stream, args);
    }
  } else {
    if (w.bK == 128) {
      if (xlds) launch_mg<128, true, false>(mode, MG, RG, w.R, mchunks, lds, stream, args);
      else launch_mg<128, false, false>(mode, MG, RG, w.R, mchunks, lds, stream, args);
    } else {
      if (xlds) launch_mg<64, true, false>(mode, MG, RG, w.R, mchunks, lds, stream, args);
      else launch_mg<64, false, false>(mode, MG, RG, w.R, mchunks, lds, stream, args);
    }
  }
  return hipGetLastError();
}

}  // namespace aq
