// Temporary INT8 operand for long prefill (AlignQuant App. E.3, Prefill: for
// a projection that holds INT4 tiles and a prompt of M' >= 1024 rows, the
// selected weights are prepared once per call as INT8 in logical tile order,
// keeping each tile's values and scales; the matrix-core schedule then reuses
// them across all activation-row groups).
//
// Output: E holds tile t = r*C + j at t * 64*b_K bytes in the INT8 tile
// layout (b_K/16 panels of [64 rows][16 codes]); Es holds its 64 FP32 row
// scales at t * 64.  One workgroup per tile: the tile's physical index comes
// from eq. 16 (row offset + same-precision tiles before it in the row); an
// INT8 tile is copied, an INT4 tile's nibbles are sign-extended to INT8
// codes (eq. 17 byte order: low nibble = column 32q + b, high nibble =
// column 32q + 16 + b of panel pair q).

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

// Four signed nibbles (one per byte, in bits 0-3) sign-extended to INT8:
// bit 3 set -> high nibble all ones.  (v & 0x08) * 0x1E = 0xF0 stays inside
// its byte, so the four bytes never interact.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t v) {
  return v | ((v & 0x08080808u) * 0x1Eu);
}

template <int BK>
__global__ __launch_bounds__(256) void expand_kernel(const PackedView w, int label_words,
                                                     int8_t *__restrict__ E,
                                                     float *__restrict__ Es) {
  constexpr int W8N = 4 * BK;  // 16-byte chunks of an INT8 tile (64 * BK / 16)
  constexpr int W4N = 2 * BK;  // 16-byte chunks of an INT4 tile
  const int t = blockIdx.x;
  const int r = t / w.C, j = t - r * w.C;
  const int is4 = tile_label(w.labels, t);
  const int before4 = count_int4(w.labels, r * w.C, j, label_words);
  const int idx = is4 ? w.off4[r] + before4 : w.off8[r] + (j - before4);
  v4i *dst = reinterpret_cast<v4i *>(E + (size_t)t * (64 * BK));
  if (is4) {
    const v4i *src = reinterpret_cast<const v4i *>(w.w4 + (size_t)idx * (32 * BK));
    for (int c = threadIdx.x; c < W4N; c += 256) {
      const v4i v = src[c];
      const int q = c >> 6, i = c & 63;
      v4i lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = (int)sext_nibbles((uint32_t)v[e] & 0x0F0F0F0Fu);
        hi[e] = (int)sext_nibbles(((uint32_t)v[e] >> 4) & 0x0F0F0F0Fu);
      }
      dst[(2 * q) * 64 + i] = lo;
      dst[(2 * q + 1) * 64 + i] = hi;
    }
  } else {
    const v4i *src = reinterpret_cast<const v4i *>(w.w8 + (size_t)idx * (64 * BK));
    for (int c = threadIdx.x; c < W8N; c += 256) dst[c] = src[c];
  }
  if (threadIdx.x < 64)
    Es[(size_t)t * 64 + threadIdx.x] = (is4 ? w.s4 : w.s8)[(size_t)idx * 64 + threadIdx.x];
}

}  // namespace

void expand_layout(const PackedView &w, const void *ws, const int8_t **E, const float **Es) {
  const int8_t *e = static_cast<const int8_t *>(ws);
  *E = e;
  *Es = reinterpret_cast<const float *>(e + (((size_t)w.N * w.K + 255) & ~(size_t)255));
}

hipError_t launch_expand(const PackedView &w, void *ws, hipStream_t stream, const int8_t **E,
                         const float **Es) {
  int8_t *e = static_cast<int8_t *>(ws);
  float *s = reinterpret_cast<float *>(e + (((size_t)w.N * w.K + 255) & ~(size_t)255));
  const int words = (w.R * w.C + 31) / 32;
  if (w.bK == 128)
    hipLaunchKernelGGL(expand_kernel<128>, dim3(w.R * w.C), dim3(256), 0, stream, w, words, e, s);
  else
    hipLaunchKernelGGL(expand_kernel<64>, dim3(w.R * w.C), dim3(256), 0, stream, w, words, e, s);
  *E = e;
  *Es = s;
  return hipGetLastError();
}

}  // namespace aq
