// Weight quantization and packing (AlignQuant App. B.2 eq. 5-6; App. E.1-E.2).
//
// One workgroup per logical tile (r, j).  BK/32 threads share a tile row;
// thread q of row i owns the 32 consecutive columns 32q .. 32q+31, which are
// exactly one INT4 panel or two INT8 panels of the packed layout, so every
// thread writes whole 16-byte chunks.  Scale and code arithmetic is FP64 with
// correctly rounded division and round-half-even, as the pages prescribe for
// integer construction.

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

constexpr int kGrid = 129;  // App. B.2 eq. 7: candidates i = 0 .. 128

// Eq. 7 squared error of one row segment at scale sc: sum over the columns
// in index order of (a - sc * Q(a; sc))^2, every product and sum rounded on
// its own (no fused multiply-add).
template <int BK>
__device__ double grid_error(const float *row, double sc, double qmin, double qmax) {
#pragma clang fp contract(off)
  double err = 0.0;
  for (int k = 0; k < BK; ++k) {
    const double a = (double)row[k];
    const double qv = fmin(fmax(rint(a / sc), qmin), qmax);
    const double d = a - sc * qv;
    err = err + d * d;
  }
  return err;
}

template <int BK, bool MSE>
__global__ __launch_bounds__(64 * (BK / 32)) void pack_kernel(
    const float *__restrict__ W, int K, int C, int label_words,
    const uint8_t *__restrict__ labels, const int32_t *__restrict__ off4,
    const int32_t *__restrict__ off8, uint8_t *__restrict__ w4, int8_t *__restrict__ w8,
    float *__restrict__ s4, float *__restrict__ s8, int T4, int T8) {
  constexpr int TPR = BK / 32;  // threads per tile row
  const int t = blockIdx.x;     // logical tile r*C + j
  const int r = t / C;
  const int j = t - r * C;
  const int i = threadIdx.x / TPR;  // row inside the tile
  const int q = threadIdx.x % TPR;  // 32-column chunk

  // Physical index, eq. 16: stored row offset + same-precision tiles before j.
  const int is4 = tile_label(labels, t);
  const int n4_before = count_int4(labels, r * C, j, label_words);
  const int idx = is4 ? off4[r] + n4_before : off8[r] + (j - n4_before);
  if (is4 ? (idx < 0 || idx >= T4) : (idx < 0 || idx >= T8)) return;  // inconsistent metadata

  const size_t n = (size_t)r * kTileRows + i;
  const float4 *src = reinterpret_cast<const float4 *>(W + n * K + (size_t)j * BK + q * 32);
  float v[32];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 f = src[e];
    v[4 * e + 0] = f.x; v[4 * e + 1] = f.y; v[4 * e + 2] = f.z; v[4 * e + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

  const double qmax = is4 ? 7.0 : 127.0;
  const double qmin = is4 ? -8.0 : -128.0;
  double s = fmax((double)amax / qmax, 1e-12);
  if constexpr (MSE) {
    // App. B.2 eq. 7: the row's scale is the first of s_i = max((1/4 + i/128)
    // s0, 1e-12), i = 0 .. 128, with the least squared error, s0 the endpoint
    // scale of eq. 6.  The tile is staged in LDS; one thread per (row, i).
    __shared__ float tv[kTileRows * BK];
    __shared__ double errs[kTileRows * kGrid];
    __shared__ double s0v[kTileRows], sst[kTileRows];
#pragma unroll
    for (int e = 0; e < 32; ++e) tv[i * BK + q * 32 + e] = v[e];
    float mx = 0.0f, mn = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      mx = fmaxf(mx, v[e]);
      mn = fminf(mn, v[e]);
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      mn = fminf(mn, __shfl_xor(mn, o));
    }
    if (q == 0) s0v[i] = fmax(fmax((double)mx / qmax, -(double)mn / -qmin), 1e-12);
    __syncthreads();
    for (int p = threadIdx.x; p < kTileRows * kGrid; p += blockDim.x) {
      const int row = p / kGrid, c = p - row * kGrid;
      const double sc = fmax((0.25 + c / 128.0) * s0v[row], 1e-12);
      errs[p] = grid_error<BK>(tv + row * BK, sc, qmin, qmax);
    }
    __syncthreads();
    if (threadIdx.x < kTileRows) {
      const int row = threadIdx.x;
      double best = errs[row * kGrid];
      int bc = 0;
      for (int c = 1; c < kGrid; ++c)
        if (errs[row * kGrid + c] < best) {
          best = errs[row * kGrid + c];
          bc = c;
        }
      sst[row] = fmax((0.25 + bc / 128.0) * s0v[row], 1e-12);
    }
    __syncthreads();
    s = sst[i];
  }
  int code[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    double c = rint((double)v[e] / s);
    c = fmin(fmax(c, qmin), qmax);
    code[e] = (int)c;
  }

  if (!is4) {
    int8_t *tile = w8 + (size_t)idx * kTileRows * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // panels 2q and 2q+1
      uint32_t word[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        word[b] = (uint32_t)(code[16 * h + 4 * b + 0] & 0xFF) |
                  ((uint32_t)(code[16 * h + 4 * b + 1] & 0xFF) << 8) |
                  ((uint32_t)(code[16 * h + 4 * b + 2] & 0xFF) << 16) |
                  ((uint32_t)(code[16 * h + 4 * b + 3] & 0xFF) << 24);
      *reinterpret_cast<uint4 *>(tile + (size_t)(2 * q + h) * kTileRows * 16 + i * 16) =
          make_uint4(word[0], word[1], word[2], word[3]);
    }
    if (q == 0) s8[(size_t)idx * kTileRows + i] = (float)s;
  } else {
    uint8_t *tile = w4 + (size_t)idx * kTileRows * BK / 2;
    uint32_t word[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t wv = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * b + e;  // byte k packs columns k (low) and k + 16 (high)
        const uint32_t byte = (uint32_t)(code[k] & 0xF) | ((uint32_t)(code[k + 16] & 0xF) << 4);
        wv |= byte << (8 * e);
      }
      word[b] = wv;
    }
    *reinterpret_cast<uint4 *>(tile + (size_t)q * kTileRows * 16 + i * 16) =
        make_uint4(word[0], word[1], word[2], word[3]);
    if (q == 0) s4[(size_t)idx * kTileRows + i] = (float)s;
  }
}

template <bool MSE>
void launch_pack_t(const float *W, const aq_packed &out, hipStream_t stream) {
  const int R = out.N / kTileRows, C = out.K / out.bK;
  const int T = R * C;
  const int label_words = (T + 31) / 32;
  if (out.bK == 128)
    hipLaunchKernelGGL((pack_kernel<128, MSE>), dim3(T), dim3(256), 0, stream, W, out.K, C, label_words,
                       out.labels, out.row_off4, out.row_off8, out.w4, out.w8, out.s4, out.s8,
                       out.T4, out.T8);
  else
    hipLaunchKernelGGL((pack_kernel<64, MSE>), dim3(T), dim3(128), 0, stream, W, out.K, C, label_words,
                       out.labels, out.row_off4, out.row_off8, out.w4, out.w8, out.s4, out.s8,
                       out.T4, out.T8);
}

}  // namespace

hipError_t launch_pack(const float *W, const aq_packed &out, hipStream_t stream, bool mse) {
  if (mse) launch_pack_t<true>(W, out, stream);
  else launch_pack_t<false>(W, out, stream);
  return hipGetLastError();
}

}  // namespace aq
