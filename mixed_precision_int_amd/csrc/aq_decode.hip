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
// Per tile a wave loads its 16 rows: two 16-byte loads per lane for an INT8
// tile (b_K = 128), one for an INT4 tile; the load addresses are selected
// without branches (an INT4 tile repeats its first address), so the loop is
// a fixed-shape software pipeline DEPTH tiles deep.  Precision labels
// (App. E.1) are read as 32-bit words into scalar registers and the physical
// tile index (eq. 16: row offset plus the same-precision tiles before it) is
// tracked in scalar registers.
//
// Products use v_mfma_i32_16x16x64_i8 with the 16 weight rows as the A
// operand and up to 16 tokens per MFMA as the B operand (tokens beyond M are
// zero).  Lane l supplies row/token l % 16 and 16 bytes of k-group g = l / 16;
// weight and activation bytes of a lane always cover the same 16 columns:
//   b_K = 128, INT8: step u, k-group g <- panel 2g+u   (columns 32g+16u ..)
//   b_K = 128, INT4: k-group g <- panel g; low nibbles feed step 0 (32g ..),
//                    high nibbles step 1 (32g+16 ..)
//   b_K =  64, INT8: k-group g <- panel g (columns 16g ..)
//   b_K =  64, INT4: k-group g <- bytes 8(g&1) .. +7 of panel g>>1: low
//                    nibbles columns 32(g>>1)+8(g&1) .., high nibbles +16
// Each tile's INT32 product is rescaled by its per-row FP32 scale into FP32
// accumulators (eq. 19).  INT4 tiles are widened x16 (see w4_lo16), so their
// scale is multiplied by the exact factor 1/16.

#include "aq_device.h"
#include "aq_internal.h"

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
  int N, K, R, C, T4, T8, M, label_words;
};

__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ uint2 load8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }

template <int BK, int MG, int WAVES, int RG, int DEPTH, bool PARTIALS>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(const DecodeArgs a) {
  constexpr int KS = BK / 64;    // MFMA steps per tile
  constexpr int S = WAVES / RG;  // splits per row group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blocks_per_row = 4 / RG;
  const int r = blockIdx.x / blocks_per_row;
  const int rgl = wave % RG;                       // row group inside the block
  const int rg = (blockIdx.x % blocks_per_row) * RG + rgl;
  const int sp = wave / RG;                        // split of this wave
  const int c0 = (a.C * sp) / S;
  const int c1 = (a.C * (sp + 1)) / S;
  const int mbase = blockIdx.y * 16 * MG;
  const int g = lane >> 4, i16 = lane & 15;
  const int rowoff = rg * 256 + i16 * 16;  // this lane's row inside a 1 KB panel
  const uint8_t *__restrict__ w4p = a.w4;
  const uint8_t *__restrict__ w8p = reinterpret_cast<const uint8_t *>(a.w8);
  const float *__restrict__ s4p = a.s4;
  const float *__restrict__ s8p = a.s8;
  const int T4 = a.T4, T8 = a.T8;

  // eq. 16 bookkeeping in scalar registers
  const int tb = r * a.C;
  const int n4 = count_int4(a.labels, tb, c0, a.label_words);
  int idx4 = a.off4[r] + n4;
  int idx8 = a.off8[r] + (c0 - n4);

  // Activation rows of this lane.  Padding tokens (m >= M) read row M-1:
  // their MFMA columns are never written out, and every load stays in bounds
  // without a branch.
  const int8_t *xrow[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int m = min(mbase + mg * 16 + i16, a.M - 1);
    xrow[mg] = a.qx + (size_t)m * a.K;
  }

  float4 F[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) F[mg] = make_float4(0.f, 0.f, 0.f, 0.f);

  // Chunks of at most 64 tile columns, whose labels sit in one 64-bit scalar
  // mask; inside a chunk, batches of DEPTH tiles: all loads of a batch are
  // issued, then its multiplies run (the other wavefronts of the CU cover
  // the latency between batches).  Past the end of the split, and on
  // inconsistent metadata, a stage re-reads a valid tile and is marked
  // dead, so every load is unconditional and in bounds.
  for (int cb = c0; cb < c1; cb += 64) {
    const int cend = min(c1, cb + 64);
    uint64_t bits = label_bits64(a.labels, tb + cb, a.label_words);
    for (int t0 = cb; t0 < cend; t0 += DEPTH) {
      v4i W[DEPTH][KS];
      v4i X[DEPTH][MG][KS];
      float4 SC[DEPTH];
      int live[DEPTH], is4v[DEPTH], jv[DEPTH];
      int last_is4 = 0, last_idx = 0;
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int j = t0 + d;
        const int lv = j < cend;
        const int lab = (int)(bits & 1u);
        bits >>= lv;
        int is4 = lv ? lab : last_is4;
        int idx = lv ? (is4 ? idx4 : idx8) : last_idx;
        idx4 += lv & is4;
        idx8 += lv & (is4 ^ 1);
        const int inb = is4 ? (idx >= 0 && idx < T4) : (idx >= 0 && idx < T8);
        if (!inb) {  // no valid tile at this index: read tile 0 of a non-empty buffer
          is4 = T4 > 0 ? 1 : 0;
          idx = 0;
        }
        last_is4 = is4;
        last_idx = idx;
        live[d] = lv & inb;
        is4v[d] = is4;
        jv[d] = lv ? j : t0;
        if (BK == 128) {
          const uint8_t *base = is4 ? w4p + (size_t)idx * 4096 : w8p + (size_t)idx * 8192;
          const int o0 = is4 ? g * 1024 : (2 * g) * 1024;
          const int o1 = is4 ? o0 : (2 * g + 1) * 1024;
          W[d][0] = load16(base + o0 + rowoff);
          W[d][KS - 1] = load16(base + o1 + rowoff);
        } else {
          // INT8: 16 bytes of panel g; INT4: 8 bytes of panel g>>1 at 8(g&1)
          const uint8_t *p = is4 ? w4p + (size_t)idx * 2048 + (g >> 1) * 1024 + rowoff + 8 * (g & 1)
                                 : w8p + (size_t)idx * 4096 + g * 1024 + rowoff;
          const uint2 lo = load8(p);
          const uint2 hi = load8(is4 ? p : p + 8);
          W[d][0] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
        }
        SC[d] = *reinterpret_cast<const float4 *>((is4 ? s4p : s8p) + (size_t)idx * 64 + rg * 16 + 4 * g);
        const int jx = jv[d];
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          const int8_t *xp = xrow[mg] + (size_t)jx * BK;
          if (BK == 128) {
#pragma unroll
            for (int u = 0; u < KS; ++u) X[d][mg][u] = load16(xp + 32 * g + 16 * u);
          } else {
            const int ca = is4 ? 32 * (g >> 1) + 8 * (g & 1) : 16 * g;
            const int cbb = is4 ? ca + 16 : ca + 8;
            const uint2 p0 = load8(xp + ca), p1 = load8(xp + cbb);
            X[d][mg][0] = v4i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y};
          }
        }
      }
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (!live[d]) continue;
        v4i op[KS];
        float4 sc = SC[d];
        if (is4v[d]) {
          const v4i w = W[d][0];
          if (BK == 128) {
            op[0] = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_lo16(w[2]), w4_lo16(w[3])};
            op[KS - 1] = v4i{w4_hi16(w[0]), w4_hi16(w[1]), w4_hi16(w[2]), w4_hi16(w[3])};
          } else {
            op[0] = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_hi16(w[0]), w4_hi16(w[1])};
          }
          sc.x *= 0.0625f; sc.y *= 0.0625f; sc.z *= 0.0625f; sc.w *= 0.0625f;
        } else {
#pragma unroll
          for (int u = 0; u < KS; ++u) op[u] = W[d][u];
        }
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < KS; ++u)
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(op[u], X[d][mg][u], acc, 0, 0, 0);
          if constexpr (PARTIALS) {
            // lane holds rows n = 64r + 16rg + 4g + e of token mbase + 16mg + i16
            const int m = mbase + mg * 16 + i16;
            if (m < a.M) {
              const size_t nb = (size_t)r * 64 + rg * 16 + 4 * g;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                a.P[((size_t)m * a.N + nb + e) * a.C + jv[d]] = is4v[d] ? (acc[e] >> 4) : acc[e];
            }
          } else {
            F[mg].x = fmaf((float)acc[0], sc.x, F[mg].x);
            F[mg].y = fmaf((float)acc[1], sc.y, F[mg].y);
            F[mg].z = fmaf((float)acc[2], sc.z, F[mg].z);
            F[mg].w = fmaf((float)acc[3], sc.w, F[mg].w);
          }
        }
      }
    }
  }

  if constexpr (!PARTIALS) {
    // ordered split reduction through LDS
    __shared__ float4 red[WAVES][MG][64];
    if (S > 1) {
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) red[wave][mg][lane] = F[mg];
      __syncthreads();
      if (sp != 0) return;
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        float4 v = red[rgl][mg][lane];
#pragma unroll
        for (int ss = 1; ss < S; ++ss) {
          const float4 p = red[ss * RG + rgl][mg][lane];
          v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        F[mg] = v;
      }
    }
    const size_t n0 = (size_t)r * 64 + rg * 16 + 4 * g;
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.bias) b = *reinterpret_cast<const float4 *>(a.bias + n0);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      const int m = mbase + mg * 16 + i16;
      if (m >= a.M) continue;
      const float sxm = a.sx[m];
      float4 v = F[mg];
      v.x = v.x * sxm + b.x; v.y = v.y * sxm + b.y; v.z = v.z * sxm + b.z; v.w = v.w * sxm + b.w;
      *reinterpret_cast<float4 *>(a.Y + (size_t)m * a.N + n0) = v;
    }
  }
}

template <int BK, int MG, int WAVES, int DEPTH, bool PARTIALS>
void launch_rg(int RG, int R, int mchunks, hipStream_t stream, const DecodeArgs &args) {
  const dim3 block(WAVES * 64);
  switch (RG) {
    case 4: hipLaunchKernelGGL((decode_kernel<BK, MG, WAVES, 4, DEPTH, PARTIALS>), dim3(R, mchunks), block, 0, stream, args); break;
    case 2: hipLaunchKernelGGL((decode_kernel<BK, MG, WAVES, 2, DEPTH, PARTIALS>), dim3(R * 2, mchunks), block, 0, stream, args); break;
    default: hipLaunchKernelGGL((decode_kernel<BK, MG, WAVES, 1, DEPTH, PARTIALS>), dim3(R * 4, mchunks), block, 0, stream, args); break;
  }
}

template <int BK, bool PARTIALS>
void launch_bk(int MG, int RG, int R, int mchunks, hipStream_t stream, const DecodeArgs &args) {
  switch (MG) {
    case 1: launch_rg<BK, 1, 16, 4, PARTIALS>(RG, R, mchunks, stream, args); break;
    case 2: launch_rg<BK, 2, 16, 3, PARTIALS>(RG, R, mchunks, stream, args); break;
    case 3: launch_rg<BK, 3, 8, 3, PARTIALS>(RG, R, mchunks, stream, args); break;
    default: launch_rg<BK, 4, 8, 3, PARTIALS>(RG, R, mchunks, stream, args); break;
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
  if (P) {
    if (w.bK == 128) launch_bk<128, true>(MG, RG, w.R, mchunks, stream, args);
    else launch_bk<64, true>(MG, RG, w.R, mchunks, stream, args);
  } else {
    if (w.bK == 128) launch_bk<128, false>(MG, RG, w.R, mchunks, stream, args);
    else launch_bk<64, false>(MG, RG, w.R, mchunks, stream, args);
  }
  return hipGetLastError();
}

}  // namespace aq
