// Compute-bound phase of the tile-aligned W4/W8 x A8 linear layer
// (AlignQuant Sec. 3.3 "Prefill weight reuse"; App. E.3, eq. 19).
//
// Workgroup = 256 threads = 4 wavefronts computing a 128 (tokens) x 128
// (outputs) block, i.e. two 64-row weight-tile rows.  Wave (wm, wn) owns the
// 64 x 64 sub-block of token half wm and weight-tile row r0 + wn, so within
// one input-tile column every wave multiplies exactly one weight tile and
// one precision.
//
// For each input-tile column j the block stages, double-buffered in LDS:
//   A: the 128 x b_K INT8 activation slab, row-major with the 16-byte chunk
//      index XOR-swizzled by (row >> 1) so that MFMA fragment reads are free
//      of bank conflicts;
//   B: both weight tiles widened to INT8, as 16-column panels [panel][n][16]
//      (the INT8 tile layout); INT4 tiles are widened x16 in registers on the
//      way in (see w4_lo16), which the rescale undoes with an exact 1/16.
// Global loads of column j+1 are issued before the MFMAs of column j.
//
// Each wave runs v_mfma_i32_32x32x32_i8 on 2 x 2 fragments per 32 columns,
// then converts the INT32 tile product to FP32 and accumulates it with the
// tile's per-row weight scale (eq. 19); the token scale and the bias are
// applied once at the end.

#include "aq_device.h"
#include "aq_internal.h"

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
};

constexpr int BM = 128;
constexpr int BN = 128;

__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

template <int BK, bool PARTIALS>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int NP = BK / 16;                // 16-byte chunks per activation row
  constexpr int A_CH = BM * NP / 256;        // activation chunks per thread
  constexpr int W8_CH = 64 * NP / 256;       // INT8 weight chunks per thread and tile
  constexpr int W4_THREADS = 64 * NP / 2;    // threads loading one INT4 tile (1 chunk each)
  constexpr int KSTEPS = BK / 32;

  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][NP * BN * 16];

  // Blocks sharing weight columns run on one XCD: hardware places block k on
  // XCD k % 8, so consecutive logical blocks are gathered per XCD.
  const int G = gridDim.x;
  const int k = blockIdx.x;
  const int per = G / 8;
  const int L = (k < per * 8) ? (k % 8) * per + k / 8 : k;
  const int bm = L % a.MB;
  const int bn = L / a.MB;
  const int m0 = bm * BM;
  const int r0 = 2 * bn;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int rw = r0 + wn;  // this wave's weight-tile row
  const bool wave_live = rw < a.R;

  // running eq. 16 indices of the two tile rows (uniform)
  int nx4[2], nx8[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int r = min(r0 + tt, a.R - 1);
    nx4[tt] = a.off4[r];
    nx8[tt] = a.off8[r];
  }

  // labels of the two tile rows for the current 64-column chunk (scalar)
  uint64_t lbits[2] = {0, 0};

  v4i ra[A_CH];
  v4i rb[2][W8_CH];
  int lab[2], idx[2];       // metadata of the column being loaded
  float scl[2];             // this lane's weight scales for the wave's tile
  int cur_lab = 0, cur_idx = 0;
  float cur_sc[2] = {0.f, 0.f};

  auto load_col = [&](int j) {
#pragma unroll
    for (int it = 0; it < A_CH; ++it) {
      const int c = it * 256 + tid;
      const int row = c / NP, p = c % NP;
      const int m = m0 + row;
      ra[it] = (m < a.M) ? ld16(a.qx + (size_t)m * a.K + (size_t)j * BK + p * 16) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int r = r0 + tt;
      if (r >= a.R) { lab[tt] = 0; idx[tt] = -1; continue; }
      if ((j & 63) == 0) lbits[tt] = label_bits64(a.labels, r * a.C + j, a.label_words);
      const int l = (int)((lbits[tt] >> (j & 63)) & 1u);
      int id = l ? nx4[tt]++ : nx8[tt]++;
      if (l ? (id >= a.T4) : (id >= a.T8)) id = -1;  // inconsistent metadata: skip
      lab[tt] = l;
      idx[tt] = id;
      if (id < 0) continue;
      if (l) {
        if (tid < W4_THREADS) rb[tt][0] = ld16(a.w4 + (size_t)id * 64 * BK / 2 + tid * 16);
      } else {
#pragma unroll
        for (int e = 0; e < W8_CH; ++e)
          rb[tt][e] = ld16(a.w8 + (size_t)id * 64 * BK + (e * 256 + tid) * 16);
      }
    }
    // scales of the wave's own tile: lane's output column n = 32 fn + (lane & 31)
    const int id = idx[wn];
    if (wave_live && id >= 0) {
      const float *sp = (lab[wn] ? a.s4 : a.s8) + (size_t)id * 64 + (lane & 31);
      const float f = lab[wn] ? 0.0625f : 1.0f;
      scl[0] = sp[0] * f;
      scl[1] = sp[32] * f;
    } else {
      scl[0] = scl[1] = 0.f;
    }
  };

  auto store_col = [&](int st) {
#pragma unroll
    for (int it = 0; it < A_CH; ++it) {
      const int c = it * 256 + tid;
      const int row = c / NP, p = c % NP;
      const int sw = p ^ ((row >> 1) & (NP - 1));
      *reinterpret_cast<v4i *>(&As[st][row * BK + sw * 16]) = ra[it];
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (idx[tt] < 0) continue;
      if (lab[tt]) {
        if (tid < W4_THREADS) {
          const int q = tid / 64, i = tid % 64;
          const v4i w = rb[tt][0];
          const v4i lo = v4i{w4_lo16(w[0]), w4_lo16(w[1]), w4_lo16(w[2]), w4_lo16(w[3])};
          const v4i hi = v4i{w4_hi16(w[0]), w4_hi16(w[1]), w4_hi16(w[2]), w4_hi16(w[3])};
          *reinterpret_cast<v4i *>(&Bs[st][((2 * q) * BN + tt * 64 + i) * 16]) = lo;
          *reinterpret_cast<v4i *>(&Bs[st][((2 * q + 1) * BN + tt * 64 + i) * 16]) = hi;
        }
      } else {
#pragma unroll
        for (int e = 0; e < W8_CH; ++e) {
          const int c = e * 256 + tid;
          const int p = c / 64, i = c % 64;
          *reinterpret_cast<v4i *>(&Bs[st][(p * BN + tt * 64 + i) * 16]) = rb[tt][e];
        }
      }
    }
  };

  v16i acc[2][2];
  float F[2][2][16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][fn][e] = 0.f;

  auto compute_col = [&](int st, int j) {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[fm][fn][e] = 0;
    const int h = lane >> 5;
#pragma unroll
    for (int u = 0; u < KSTEPS; ++u) {
      const int p = 2 * u + h;
      v4i af[2], bf[2];
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        const int row = wm * 64 + fm * 32 + (lane & 31);
        const int sw = p ^ ((row >> 1) & (NP - 1));
        af[fm] = *reinterpret_cast<const v4i *>(&As[st][row * BK + sw * 16]);
      }
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const int n = wn * 64 + fn * 32 + (lane & 31);
        bf[fn] = *reinterpret_cast<const v4i *>(&Bs[st][(p * BN + n) * 16]);
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
    }
    if constexpr (PARTIALS) {
      // C layout of the 32x32 MFMA: column (output n) = lane & 31,
      // row (token) = 8 (e / 4) + 4 (lane >> 5) + (e & 3).
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * 64 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3);
            const size_t n = (size_t)rw * 64 + fn * 32 + (lane & 31);
            if (m < a.M) {
              const int v = acc[fm][fn][e];
              a.P[((size_t)m * a.N + n) * a.C + j] = cur_lab ? (v >> 4) : v;
            }
          }
    } else {
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            F[fm][fn][e] = fmaf((float)acc[fm][fn][e], cur_sc[fn], F[fm][fn][e]);
    }
  };

  load_col(0);
  store_col(0);
  cur_lab = lab[wn]; cur_idx = idx[wn]; cur_sc[0] = scl[0]; cur_sc[1] = scl[1];
  __syncthreads();
  for (int j = 0; j < a.C; ++j) {
    const int st = j & 1;
    const bool more = j + 1 < a.C;
    if (more) load_col(j + 1);
    if (wave_live && cur_idx >= 0) compute_col(st, j);
    if (more) {
      store_col(st ^ 1);
      cur_lab = lab[wn]; cur_idx = idx[wn]; cur_sc[0] = scl[0]; cur_sc[1] = scl[1];
    }
    __syncthreads();
  }

  if constexpr (!PARTIALS) {
    if (!wave_live) return;
    const int h = lane >> 5;
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

template <int BK>
void launch_bk(bool partials, dim3 grid, hipStream_t stream, const PrefillArgs &args) {
  if (partials)
    hipLaunchKernelGGL((prefill_kernel<BK, true>), grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((prefill_kernel<BK, false>), grid, dim3(256), 0, stream, args);
}

}  // namespace

hipError_t launch_prefill(const PackedView &w, const int8_t *qx, const float *sx, int M,
                          const float *bias, float *Y, int32_t *P, hipStream_t stream) {
  PrefillArgs args;
  args.labels = w.labels; args.off4 = w.off4; args.off8 = w.off8;
  args.w4 = w.w4; args.w8 = w.w8; args.s4 = w.s4; args.s8 = w.s8;
  args.qx = qx; args.sx = sx; args.bias = bias; args.Y = Y; args.P = P;
  args.N = w.N; args.K = w.K; args.R = w.R; args.C = w.C; args.T4 = w.T4; args.T8 = w.T8;
  args.M = M;
  args.label_words = (w.R * w.C + 31) / 32;
  args.MB = (M + BM - 1) / BM;
  args.NB = (w.R + 1) / 2;
  const dim3 grid(args.MB * args.NB);
  if (w.bK == 128) launch_bk<128>(P != nullptr, grid, stream, args);
  else launch_bk<64>(P != nullptr, grid, stream, args);
  return hipGetLastError();
}

}  // namespace aq
