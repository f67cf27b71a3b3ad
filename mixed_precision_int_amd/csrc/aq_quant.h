// Per-token activation quantization (AlignQuant App. B.3 with App. B.2
// eq. 5): device helpers shared by the plain and the transformed quantizers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

// code = clip(rint(x / s), -128, 127), FP64 division (correctly rounded),
// rint ties to even.
__device__ __forceinline__ uint32_t code_of(float x, double s) {
  double q = rint((double)x / s);
  q = fmin(fmax(q, -128.0), 127.0);
  return (uint32_t)((int)q & 0xFF);
}

__device__ __forceinline__ uint32_t codes4(const float4 &v, double s) {
  return code_of(v.x, s) | (code_of(v.y, s) << 8) | (code_of(v.z, s) << 16) |
         (code_of(v.w, s) << 24);
}

// code_of(x, s) with the FP64 division taken only where an FP32 estimate
// cannot decide it.  inv = 1/s rounded to FP32 (from the FP64 reciprocal),
// p = x * inv rounded to FP32, so p = (x / s)(1 + d) with |d| < 2^-23 +
// 2^-47.  The estimate is used when r = rint(p) has |r| <= 127 and
// |p - r| < 1/2 - 2^-15: then |x / s| < 128, |p - x / s| < 2^-16 + 2^-40,
// and x / s lies inside (r - 1/2 + 2^-17, r + 1/2 - 2^-17); its FP64
// quotient (within 2^-46 of it) rounds to r too, and r needs no clipping.
// Every other case (near ties, out of range, NaN) takes code_of.
__device__ __forceinline__ uint32_t code_fast(float x, double s, float inv) {
  const float p = x * inv;
  const float r = rintf(p);
  if (fabsf(p - r) < 0.5f - 0x1p-15f && fabsf(r) <= 127.0f) return (uint32_t)((int)r & 0xFF);
  return code_of(x, s);
}

__device__ __forceinline__ uint32_t codes4_fast(const float4 &v, double s, float inv) {
  return code_fast(v.x, s, inv) | (code_fast(v.y, s, inv) << 8) | (code_fast(v.z, s, inv) << 16) |
         (code_fast(v.w, s, inv) << 24);
}

// Bits of |x|: for non-negative IEEE floats the unsigned order of the bit
// patterns is the numeric order, so the maximum is an integer max.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t abs_bits4(const float4 &v) {
  return max(max(abs_bits(v.x), abs_bits(v.y)), max(abs_bits(v.z), abs_bits(v.w)));
}

// Maximum over the 64 lanes of a wavefront, returned uniform.  DPP within
// rows of 16 lanes (quad xor 1, quad xor 2, half-row mirror, row mirror),
// ds_swizzle across the two rows of each 32-lane half, then the two halves.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  return max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
             (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}

// Row maximum across the T/64 waves of the workgroup.
template <int T>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[T / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) r = max(r, red[w]);
  return r;
}

// Scale of the App. B.3 rule: s = max(max|x| / 127, 1e-12), FP64.
__device__ __forceinline__ double row_scale(uint32_t amax_bits) {
  return fmax((double)__uint_as_float(amax_bits) / 127.0, 1e-12);
}

}  // namespace aq
