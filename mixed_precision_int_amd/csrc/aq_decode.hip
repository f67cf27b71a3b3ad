// Memory-bound phase of the tile-aligned W4/W8 x A8 linear layer
// (AlignQuant Sec. 3.3 "Decode parallelism"; App. E.3, Table 5, eq. 19).
//
// Work unit = one wavefront = (output-tile row r, split s).  Split s covers
// input-tile columns floor(C*s/S) .. floor(C*(s+1)/S)-1 (App. E.3).  The four
// wavefronts of a workgroup take four consecutive units, i.e. neighbouring
// splits of one tile row, so a workgroup streams one contiguous stretch of
// each packed buffer.
//
// Inside a unit the wave walks the INT8 tiles of its columns, then the INT4
// tiles (each precision is a contiguous run of its own buffer, eq. 16), so the
// inner loops are branch-free and software-pipelined one tile ahead: the
// 16-byte loads of tile t+1 are in flight while tile t is multiplied.
//
// Products use v_mfma_i32_16x16x64_i8 with the weight tile rows as the A
// operand (16 rows per row group, 4 row groups per 64-row tile) and up to 16
// tokens per MFMA as the B operand; tokens beyond M are zero.  Lane l of the
// wave supplies row/token l % 16 and 16 bytes of k-group l / 16, and for every
// tile the k-group of a lane is chosen so that the weight and activation
// bytes it loads cover the same 16 input columns:
//   b_K = 128, INT8: MFMA step u, k-group g <- panel 2g+u   (columns 32g+16u ..)
//   b_K = 128, INT4: k-group g <- panel g; low nibbles feed step 0 (32g ..),
//                    high nibbles step 1 (32g+16 ..)
//   b_K =  64, INT8: k-group g <- panel g (columns 16g ..)
//   b_K =  64, INT4: k-group g <- bytes 8(g&1) .. +7 of panel g>>1: low
//                    nibbles columns 32(g>>1)+8(g&1) .., high nibbles +16
// Each tile's INT32 product is rescaled by its per-row FP32 scale and added to
// FP32 accumulators (eq. 19).  INT4 tiles are widened x16 (see w4_lo16), so
// their scale is multiplied by 1/16, which is exact.

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
  float *Y, *ws;
  int32_t *P;
  int N, K, R, C, T4, T8, M, S, labels_bytes;
};

__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ uint2 load8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }

template <int BK, int MG>
struct Act {
  static constexpr int KS = BK / 64;  // MFMA steps per row group
  v4i x[MG][KS];
};

// Activation fragments of tile column j for an INT8 tile (and for INT4 tiles
// when b_K = 128, where both precisions use the same columns per lane).
template <int BK, int MG>
__device__ __forceinline__ void load_act_std(Act<BK, MG> &A, const int8_t *__restrict__ qx, int K,
                                             int M, int mbase, int lane, int j) {
  const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int m = mbase + mg * 16 + i16;
    const int8_t *row = qx + (size_t)m * K + (size_t)j * BK;
#pragma unroll
    for (int u = 0; u < Act<BK, MG>::KS; ++u) {
      const int col = (BK == 128) ? (32 * g + 16 * u) : (16 * g);
      A.x[mg][u] = (m < M) ? load16(row + col) : v4i{0, 0, 0, 0};
    }
  }
}

// b_K = 64 INT4 tile: columns 32p + 8h + (0..7) and 32p + 16 + 8h + (0..7),
// p = g >> 1, h = g & 1.
template <int MG>
__device__ __forceinline__ void load_act_w4_bk64(Act<64, MG> &A, const int8_t *__restrict__ qx,
                                                 int K, int M, int mbase, int lane, int j) {
  const int g = lane >> 4, i16 = lane & 15;
  const int col = 32 * (g >> 1) + 8 * (g & 1);
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int m = mbase + mg * 16 + i16;
    const int8_t *row = qx + (size_t)m * K + (size_t)j * 64;
    if (m < M) {
      const uint2 a = load8(row + col), b = load8(row + col + 16);
      A.x[mg][0] = v4i{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
    } else {
      A.x[mg][0] = v4i{0, 0, 0, 0};
    }
  }
}

template <int BK, int MG>
struct Tile8 {
  static constexpr int KS = BK / 64;
  v4i w[4][KS];
  float4 sc[4];
  Act<BK, MG> a;
};

template <int BK, int MG>
struct Tile4 {
  // b_K = 128: 16 bytes (one 32-column panel) per lane and row group;
  // b_K = 64: 8 bytes per lane and row group, kept in .x/.y.
  v4i w[4];
  float4 sc[4];
  Act<BK, MG> a;
};

template <int BK, int MG, bool PARTIALS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int KS = BK / 64;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.R * a.S) return;
  const int r = unit / a.S;
  const int s = unit - r * a.S;
  const int c0 = (int)(((long long)a.C * s) / a.S);
  const int c1 = (int)(((long long)a.C * (s + 1)) / a.S);
  const int mbase = blockIdx.y * 16 * MG;
  const int g = lane >> 4, i16 = lane & 15;
  const int rowoff = i16 * 16;  // byte offset of this lane's tile row in a panel

  float4 F[4][MG];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) F[rg][mg] = make_float4(0.f, 0.f, 0.f, 0.f);

  // P[m, n, j] for the debug mode: lane holds rows n = r*64 + 16rg + 4g + e,
  // token m = mbase + 16mg + i16.
  auto write_partials = [&](int rg, int mg, v4i acc, int j, bool w4tile) {
    const int m = mbase + mg * 16 + i16;
    if (m >= a.M) return;
    const size_t nb = (size_t)r * 64 + rg * 16 + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = w4tile ? (acc[e] >> 4) : acc[e];
      a.P[((size_t)m * a.N + nb + e) * a.C + j] = v;
    }
  };

  auto accumulate = [&](int rg, int mg, v4i acc, float4 sc) {
    F[rg][mg].x = fmaf((float)acc[0], sc.x, F[rg][mg].x);
    F[rg][mg].y = fmaf((float)acc[1], sc.y, F[rg][mg].y);
    F[rg][mg].z = fmaf((float)acc[2], sc.z, F[rg][mg].z);
    F[rg][mg].w = fmaf((float)acc[3], sc.w, F[rg][mg].w);
  };

  // ---- INT8 tiles
  auto load8t = [&](Tile8<BK, MG> &T, int j, int idx) {
    const int8_t *tile = a.w8 + (size_t)idx * 64 * BK;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const int panel = (BK == 128) ? (2 * g + u) : g;
        T.w[rg][u] = load16(tile + panel * 1024 + rg * 256 + rowoff);
      }
    const float *sc = a.s8 + (size_t)idx * 64 + 4 * g;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) T.sc[rg] = *reinterpret_cast<const float4 *>(sc + rg * 16);
    load_act_std<BK, MG>(T.a, a.qx, a.K, a.M, mbase, lane, j);
  };
  auto comp8t = [&](Tile8<BK, MG> &T, int j) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < KS; ++u)
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(T.w[rg][u], T.a.x[mg][u], acc, 0, 0, 0);
        if constexpr (PARTIALS) write_partials(rg, mg, acc, j, false);
        else accumulate(rg, mg, acc, T.sc[rg]);
      }
  };

  // ---- INT4 tiles
  auto load4t = [&](Tile4<BK, MG> &T, int j, int idx) {
    const uint8_t *tile = a.w4 + (size_t)idx * 64 * BK / 2;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      if constexpr (BK == 128) {
        T.w[rg] = load16(tile + g * 1024 + rg * 256 + rowoff);
      } else {
        const uint2 v = load8(tile + (g >> 1) * 1024 + rg * 256 + rowoff + 8 * (g & 1));
        T.w[rg] = v4i{(int)v.x, (int)v.y, 0, 0};
      }
    }
    const float *sc = a.s4 + (size_t)idx * 64 + 4 * g;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) T.sc[rg] = *reinterpret_cast<const float4 *>(sc + rg * 16);
    if constexpr (BK == 128) load_act_std<BK, MG>(T.a, a.qx, a.K, a.M, mbase, lane, j);
    else load_act_w4_bk64<MG>(T.a, a.qx, a.K, a.M, mbase, lane, j);
  };
  auto comp4t = [&](Tile4<BK, MG> &T, int j) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      v4i op[KS];
      const v4i w = T.w[rg];
      if constexpr (BK == 128) {
        op[0] = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_lo16(w[2]), w4_lo16(w[3])};
        op[1] = v4i{w4_hi16(w[0]), w4_hi16(w[1]), w4_hi16(w[2]), w4_hi16(w[3])};
      } else {
        op[0] = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_hi16(w[0]), w4_hi16(w[1])};
      }
      const float4 sc = make_float4(T.sc[rg].x * 0.0625f, T.sc[rg].y * 0.0625f,
                                    T.sc[rg].z * 0.0625f, T.sc[rg].w * 0.0625f);
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < KS; ++u)
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(op[u], T.a.x[mg][u], acc, 0, 0, 0);
        if constexpr (PARTIALS) write_partials(rg, mg, acc, j, true);
        else accumulate(rg, mg, acc, sc);
      }
    }
  };

  // Walk the set bits of `mask` (tile columns cc + bit) in increasing order,
  // one tile of loads ahead of the multiplies.
  auto run = [&](auto &bufA, auto &bufB, uint32_t mask, int cc, int idx, auto load, auto comp) {
    if (!mask) return;
    int j = cc + __builtin_ctz(mask);
    mask &= mask - 1;
    load(bufA, j, idx);
    while (true) {
      if (!mask) { comp(bufA, j); return; }
      const int jn = cc + __builtin_ctz(mask);
      mask &= mask - 1;
      load(bufB, jn, idx + 1);
      comp(bufA, j);
      ++idx;
      if (!mask) { comp(bufB, jn); return; }
      j = cc + __builtin_ctz(mask);
      mask &= mask - 1;
      load(bufA, j, idx + 1);
      comp(bufB, jn);
      ++idx;
    }
  };

  const int tb = r * a.C;
  const int n4 = count_int4(a.labels, tb, c0, a.labels_bytes);
  int idx4 = a.off4[r] + n4;
  int idx8 = a.off8[r] + (c0 - n4);

  for (int cc = c0; cc < c1; cc += 32) {
    const int nb = min(32, c1 - cc);
    const uint32_t valid = nb == 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u);
    const uint32_t bits = label_bits32(a.labels, tb + cc, a.labels_bytes);
    const uint32_t m4 = bits & valid, m8 = ~bits & valid;
    const int k4 = __popc(m4), k8 = __popc(m8);
    // Inconsistent metadata would index past a buffer: such tiles are skipped.
    if (idx8 >= 0 && idx8 + k8 <= a.T8) {
      Tile8<BK, MG> A8, B8;
      run(A8, B8, m8, cc, idx8, load8t, comp8t);
    }
    if (idx4 >= 0 && idx4 + k4 <= a.T4) {
      Tile4<BK, MG> A4, B4;
      run(A4, B4, m4, cc, idx4, load4t, comp4t);
    }
    idx8 += k8;
    idx4 += k4;
  }

  if constexpr (!PARTIALS) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const int m = mbase + mg * 16 + i16;
        if (m >= a.M) continue;
        const size_t n0 = (size_t)r * 64 + rg * 16 + 4 * g;
        float4 v = F[rg][mg];
        if (a.S == 1) {
          const float sxm = a.sx[m];
          v.x *= sxm; v.y *= sxm; v.z *= sxm; v.w *= sxm;
          if (a.bias) {
            const float4 b = *reinterpret_cast<const float4 *>(a.bias + n0);
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
          }
          *reinterpret_cast<float4 *>(a.Y + (size_t)m * a.N + n0) = v;
        } else {
          *reinterpret_cast<float4 *>(a.ws + ((size_t)s * a.M + m) * a.N + n0) = v;
        }
      }
  }
}

// Y[m, n] = sx[m] * sum_{s = 0..S-1} ws[s, m, n] (+ bias[n]); splits summed in
// increasing order (App. E.3).  One thread per 4 consecutive outputs.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ ws, int S,
                                                           int M, int N,
                                                           const float *__restrict__ sx,
                                                           const float *__restrict__ bias,
                                                           float *__restrict__ Y) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n4 = N / 4;
  if (q >= (size_t)M * n4) return;
  const size_t m = q / n4;
  const size_t n0 = (q - m * n4) * 4;
  const size_t plane = (size_t)M * N;
  const float4 *src = reinterpret_cast<const float4 *>(ws + m * N + n0);
  float4 acc = src[0];
  for (int s = 1; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4 *>(ws + s * plane + m * N + n0);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const float sxm = sx[m];
  acc.x *= sxm; acc.y *= sxm; acc.z *= sxm; acc.w *= sxm;
  if (bias) {
    const float4 b = *reinterpret_cast<const float4 *>(bias + n0);
    acc.x += b.x; acc.y += b.y; acc.z += b.z; acc.w += b.w;
  }
  *reinterpret_cast<float4 *>(Y + m * N + n0) = acc;
}

template <int BK, bool PARTIALS>
void launch_bk(int MG, dim3 grid, hipStream_t stream, const DecodeArgs &args) {
  switch (MG) {
    case 1: hipLaunchKernelGGL((decode_kernel<BK, 1, PARTIALS>), grid, dim3(256), 0, stream, args); break;
    case 2: hipLaunchKernelGGL((decode_kernel<BK, 2, PARTIALS>), grid, dim3(256), 0, stream, args); break;
    case 3: hipLaunchKernelGGL((decode_kernel<BK, 3, PARTIALS>), grid, dim3(256), 0, stream, args); break;
    default: hipLaunchKernelGGL((decode_kernel<BK, 4, PARTIALS>), grid, dim3(256), 0, stream, args); break;
  }
}

}  // namespace

int decode_split(const PackedView &w, int M) {
  (void)M;
  // Enough wavefronts in flight to cover HBM latency on 256 CUs: about
  // eight per CU, never more splits than tile columns.
  const int target_units = 2048;
  int S = (target_units + w.R - 1) / w.R;
  if (S > w.C) S = w.C;
  if (S < 1) S = 1;
  return S;
}

hipError_t launch_decode(const PackedView &w, const int8_t *qx, const float *sx, int M,
                         const float *bias, float *Y, int S, float *ws, int32_t *P,
                         hipStream_t stream) {
  DecodeArgs args;
  args.labels = w.labels; args.off4 = w.off4; args.off8 = w.off8;
  args.w4 = w.w4; args.w8 = w.w8; args.s4 = w.s4; args.s8 = w.s8;
  args.qx = qx; args.sx = sx; args.bias = bias;
  args.Y = Y; args.ws = ws; args.P = P;
  args.N = w.N; args.K = w.K; args.R = w.R; args.C = w.C; args.T4 = w.T4; args.T8 = w.T8;
  args.M = M; args.S = P ? 1 : S; args.labels_bytes = (w.R * w.C + 7) / 8;

  const int MG = M >= 49 ? 4 : (M + 15) / 16;
  const int mchunks = (M + 16 * MG - 1) / (16 * MG);
  const dim3 grid((w.R * args.S + 3) / 4, mchunks);
  if (P) {
    if (w.bK == 128) launch_bk<128, true>(MG, grid, stream, args);
    else launch_bk<64, true>(MG, grid, stream, args);
    return hipGetLastError();
  }
  if (w.bK == 128) launch_bk<128, false>(MG, grid, stream, args);
  else launch_bk<64, false>(MG, grid, stream, args);
  if (args.S > 1) {
    const size_t quads = (size_t)M * (w.N / 4);
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, ws, args.S, M, w.N, sx, bias, Y);
  }
  return hipGetLastError();
}

}  // namespace aq
