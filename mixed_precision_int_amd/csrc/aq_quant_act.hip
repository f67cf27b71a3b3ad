// Per-token INT8 activation quantization (AlignQuant App. B.3: preparation
// computes in FP64 and stores signed INT8 codes with FP32 scales; rounding
// per App. B.2 eq. 5).  One workgroup of 256 threads per token row:
//   pass 1: |x| max over the row (float4 loads, wavefront butterfly, then
//           the four wave results through LDS);
//   pass 2: codes = clip(rint(x / s), -128, 127) with s in FP64, 16 codes per
//           thread per step written as one 16-byte store.
// The row is read twice; the second read hits the cache for the row sizes of
// the workloads (<= 70 KB per row).

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, double s) {
  const float in[4] = {a, b, c, d};
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    double q = rint((double)in[e] / s);
    q = fmin(fmax(q, -128.0), 127.0);
    w |= ((uint32_t)((int)q & 0xFF)) << (8 * e);
  }
  return w;
}

__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ X, int K,
                                                        int8_t *__restrict__ qx,
                                                        float *__restrict__ sx) {
  const size_t m = blockIdx.x;
  const float4 *row = reinterpret_cast<const float4 *>(X + m * K);
  float amax = 0.0f;
  for (int c = threadIdx.x; c < K / 4; c += 256) {
    const float4 v = row[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float red[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const double s = fmax((double)amax / 127.0, 1e-12);
  if (threadIdx.x == 0) sx[m] = (float)s;

  uint4 *out = reinterpret_cast<uint4 *>(qx + m * K);
  for (int c = threadIdx.x; c < K / 16; c += 256) {
    const float4 a = row[4 * c + 0], b = row[4 * c + 1], d = row[4 * c + 2], e = row[4 * c + 3];
    out[c] = make_uint4(quant4(a.x, a.y, a.z, a.w, s), quant4(b.x, b.y, b.z, b.w, s),
                        quant4(d.x, d.y, d.z, d.w, s), quant4(e.x, e.y, e.z, e.w, s));
  }
}

}  // namespace

hipError_t launch_quant_act(const float *X, int M, int K, int8_t *qx, float *sx,
                            hipStream_t stream) {
  hipLaunchKernelGGL(quant_act_kernel, dim3(M), dim3(256), 0, stream, X, K, qx, sx);
  return hipGetLastError();
}

}  // namespace aq
