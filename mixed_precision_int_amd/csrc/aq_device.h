// Device helpers shared by the gfx950 kernels: precision labels, physical
// tile indices and INT4 widening.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Label of logical tile t: 1 = INT4, 0 = INT8; bit (t & 7) of byte t >> 3
// (AlignQuant App. E.1 label order, first label in the least significant bit).
__device__ __forceinline__ int tile_label(const uint8_t *__restrict__ labels, int t) {
  return (labels[t >> 3] >> (t & 7)) & 1;
}

// The device label buffer is padded with zero bytes to nwords = ceil(T/32)
// 32-bit words, so labels are read as whole words (scalar loads when the
// index is uniform).  Word w holds the labels of tiles 32w .. 32w+31.
__device__ __forceinline__ uint32_t label_word(const uint8_t *__restrict__ labels, int nwords, int w) {
  return (w >= 0 && w < nwords) ? reinterpret_cast<const uint32_t *>(labels)[w] : 0u;
}

// Labels of tiles t .. t+31 (bit k = tile t + k); zero past the end.
__device__ __forceinline__ uint32_t label_bits32(const uint8_t *__restrict__ labels, int t,
                                                 int nwords) {
  const int w = t >> 5, sh = t & 31;
  const uint32_t lo = label_word(labels, nwords, w);
  if (sh == 0) return lo;
  return (lo >> sh) | (label_word(labels, nwords, w + 1) << (32 - sh));
}

// Labels of tiles t .. t+63.
__device__ __forceinline__ uint64_t label_bits64(const uint8_t *__restrict__ labels, int t,
                                                 int nwords) {
  return (uint64_t)label_bits32(labels, t, nwords) |
         ((uint64_t)label_bits32(labels, t + 32, nwords) << 32);
}

// Number of INT4 labels among tiles [t0, t0 + n).
__device__ __forceinline__ int count_int4(const uint8_t *__restrict__ labels, int t0, int n,
                                          int nwords) {
  int c = 0;
  for (int k = 0; k < n; k += 32) {
    uint32_t bits = label_bits32(labels, t0 + k, nwords);
    const int left = n - k;
    if (left < 32) bits &= (1u << left) - 1u;
    c += __popc(bits);
  }
  return c;
}

// INT4 widening, scaled by 16.  A 32-bit word of the packed tile holds four
// bytes, each byte two signed nibbles (App. E.1 eq. 17: low nibble q0, high
// nibble q1).  Masking the high nibble in place gives the int8 value 16*q1;
// shifting the low nibble up gives 16*q0.  Both are exact two's-complement
// int8 values, so a dot product over them is exactly 16x the dot product over
// the codes, and the caller divides by 16 (an exact shift or a power-of-two
// scale).  Two bit operations replace a full sign extension.
__device__ __forceinline__ int w4_lo16(uint32_t w) { return (int)((w << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int w4_hi16(uint32_t w) { return (int)(w & 0xF0F0F0F0u); }

}  // namespace aq
