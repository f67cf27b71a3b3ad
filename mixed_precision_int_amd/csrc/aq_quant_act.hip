// Per-token INT8 activation quantization (AlignQuant App. B.3: preparation
// computes in FP64 and stores signed INT8 codes with FP32 scales; rounding
// per App. B.2 eq. 5).
//
// One workgroup per token row.  The row is read once into registers (NV
// float4 per thread, coalesced 16-byte loads), its |x| maximum is reduced
// across the wavefront with DPP row permutes and one ds_swizzle, then across
// the waves through LDS; each thread then writes the INT8 codes of its own
// float4 groups as 4-byte stores (an FP32 estimate of x / s decides most codes,
// the FP64 division the rest).  Decode-sized batches (few rows) take 1024
// threads per row; prefill-sized batches take 256 threads per row and fill
// the chip with rows.  Rows longer
// than the register-resident variants cover fall back to a two-pass loop.

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_quant.h"

namespace aq {
namespace {

template <int T, int NV>
__global__ __launch_bounds__(T) void quant_act_kernel(const float *__restrict__ X, int K,
                                                      int8_t *__restrict__ qx,
                                                      float *__restrict__ sx) {
  const size_t m = blockIdx.x;
  const int n4 = K >> 2;
  const float4 *row = reinterpret_cast<const float4 *>(X + m * K);
  float4 v[NV];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * T;
    v[i] = c < n4 ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    amax = max(amax, abs_bits4(v[i]));
  }
  const double s = row_scale(block_max_u32<T>(amax));
  if (threadIdx.x == 0) sx[m] = (float)s;
  // codes by the FP32 estimate where it decides them, else the FP64 rule
  // (code_fast: the same codes as the FP64 division, bit for bit)
  const float inv = (float)(1.0 / s);
  uint32_t *out = reinterpret_cast<uint32_t *>(qx + m * K);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * T;
    if (c < n4) out[c] = codes4_fast(v[i], s, inv);
  }
}

// Any row length (K a multiple of 64): two passes over the row.
__global__ __launch_bounds__(256) void quant_act_loop_kernel(const float *__restrict__ X, int K,
                                                             int8_t *__restrict__ qx,
                                                             float *__restrict__ sx) {
  const size_t m = blockIdx.x;
  const int n4 = K >> 2;
  const float4 *row = reinterpret_cast<const float4 *>(X + m * K);
  uint32_t amax = 0;
  for (int c = threadIdx.x; c < n4; c += 256) amax = max(amax, abs_bits4(row[c]));
  const double s = row_scale(block_max_u32<256>(amax));
  if (threadIdx.x == 0) sx[m] = (float)s;
  const float inv = (float)(1.0 / s);
  uint32_t *out = reinterpret_cast<uint32_t *>(qx + m * K);
  for (int c = threadIdx.x; c < n4; c += 256) out[c] = codes4_fast(row[c], s, inv);
}

// The pages' grouping (App. B.3): one wave per group of 64 features x BM
// rows (BM = 1 for a single token, else 16; rows past M are the zero
// padding, which eq. 6's max(0, .) terms already cover).  Lane l holds
// feature 64c + l of every row of the group; the group's maximum and minimum
// are reduced across the wave; the scale is eq. 6 at 8 bits,
// s = max(max(0, max A) / 127, max(0, -min A) / 128, 1e-12) in FP64, and the
// codes are eq. 5's clip(rint(x / s), -128, 127) in FP64 (by code_fast: an
// FP32 estimate where it decides the code, the FP64 division otherwise).
template <int BM>
__global__ __launch_bounds__(256) void quant_act_grouped_kernel(const float *__restrict__ X, int M,
                                                                int K, int8_t *__restrict__ qx,
                                                                float *__restrict__ sxg) {
  const int lane = threadIdx.x & 63;
  const int kg = K >> 6;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);  // feature group (wave-uniform)
  if (c >= kg) return;
  const int r0 = blockIdx.y * BM;
  const int nr = min(BM, M - r0);
  const size_t col = (size_t)c * 64 + lane;
  float v[BM];
  float mx = 0.f, mn = 0.f;  // max(0, max A) and -max(0, -min A)
#pragma unroll
  for (int r = 0; r < BM; ++r) {
    v[r] = r < nr ? X[(size_t)(r0 + r) * K + col] : 0.f;
    mx = fmaxf(mx, v[r]);
    mn = fminf(mn, v[r]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    mn = fminf(mn, __shfl_xor(mn, o));
  }
  const double s = fmax(fmax((double)mx / 127.0, -(double)mn / 128.0), 1e-12);
  if (lane == 0) sxg[(size_t)blockIdx.y * kg + c] = (float)s;
  const float inv = (float)(1.0 / s);  // code_fast: the FP64 rule's codes (-128 always takes it)
#pragma unroll
  for (int r = 0; r < BM; ++r)
    if (r < nr) qx[(size_t)(r0 + r) * K + col] = (int8_t)(code_fast(v[r], s, inv) & 0xFF);
}

template <int T, int NV>
hipError_t launch_rows(const float *X, int M, int K, int8_t *qx, float *sx, hipStream_t stream) {
  hipLaunchKernelGGL((quant_act_kernel<T, NV>), dim3(M), dim3(T), 0, stream, X, K, qx, sx);
  return hipGetLastError();
}

// Register-resident variants: float4 groups per thread.
template <int T>
hipError_t launch_t(int nv, const float *X, int M, int K, int8_t *qx, float *sx,
                    hipStream_t stream) {
  switch (nv) {
    case 1: return launch_rows<T, 1>(X, M, K, qx, sx, stream);
    case 2: return launch_rows<T, 2>(X, M, K, qx, sx, stream);
    case 3: return launch_rows<T, 3>(X, M, K, qx, sx, stream);
    case 4: return launch_rows<T, 4>(X, M, K, qx, sx, stream);
    case 5: return launch_rows<T, 5>(X, M, K, qx, sx, stream);
    case 6: return launch_rows<T, 6>(X, M, K, qx, sx, stream);
    case 8: return launch_rows<T, 8>(X, M, K, qx, sx, stream);
    case 12: return launch_rows<T, 12>(X, M, K, qx, sx, stream);
    case 16: return launch_rows<T, 16>(X, M, K, qx, sx, stream);
    case 20: return launch_rows<T, 20>(X, M, K, qx, sx, stream);
    default: return hipErrorInvalidValue;
  }
}

int round_nv(int need) {
  static const int kNV[] = {1, 2, 3, 4, 5, 6, 8, 12, 16, 20};
  for (int v : kNV)
    if (v >= need) return v;
  return 0;
}

}  // namespace

hipError_t launch_quant_act(const float *X, int M, int K, int8_t *qx, float *sx,
                            hipStream_t stream) {
  const int n4 = K / 4;
  // Few rows: a wide workgroup per row (16 waves).  With 4 waves the
  // decode-sized rows measured the same (K = 3072: 4.59 against 4.64 us;
  // K = 8192: 4.55 against 4.53 us): the call is one load round trip and the
  // launch, not the lanes' arithmetic.
  if (M < 256) {
    const int nv = round_nv((n4 + 1023) / 1024);
    if (nv && nv <= 8) return launch_t<1024>(nv, X, M, K, qx, sx, stream);
  } else {
    const int nv = round_nv((n4 + 255) / 256);
    if (nv) return launch_t<256>(nv, X, M, K, qx, sx, stream);
  }
  hipLaunchKernelGGL(quant_act_loop_kernel, dim3(M), dim3(256), 0, stream, X, K, qx, sx);
  return hipGetLastError();
}

hipError_t launch_quant_act_grouped(const float *X, int M, int K, int8_t *qx, float *sxg,
                                    hipStream_t stream) {
  const dim3 block(256);
  const int gx = (K / kActGroupK + 3) / 4;
  const int bM = act_group_rows(M);
  if (bM == 1)
    hipLaunchKernelGGL(quant_act_grouped_kernel<1>, dim3(gx, M), block, 0, stream, X, M, K, qx, sxg);
  else
    hipLaunchKernelGGL(quant_act_grouped_kernel<16>, dim3(gx, (M + 15) / 16), block, 0, stream, X, M, K,
                       qx, sxg);
  return hipGetLastError();
}

}  // namespace aq
