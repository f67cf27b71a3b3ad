// The output transform of App. B.1 (Y = Y~ U, U_r = Phi_{u_r}^T on the 64
// outputs of tile row r, eq. 4) in the epilogue of the long-prompt GEMMs,
// on their 32 x 32 MFMA accumulator layout: one token's 64 outputs of a
// tile row sit in one half-wave, output 32 fn + l32 in register fn of lane
// l32, so a wave that owns one tile row transforms every token it holds at
// once.  Shared by the short-prompt, the 256 x 128 and the persistent
// 256 x 256 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aq_internal.h"

namespace aq {

// The six signed permutations: perm rows and sign masks (bit i set:
// element i negated), one 32-bit word per half of the block (bit l of word
// f is set where element 32 f + l is flipped).
struct OutTables {
  uint8_t perm[kTransformSeeds][64];
  uint32_t dlm[kTransformSeeds][2], drm[kTransformSeeds][2];
};

inline OutTables out_tables(const TransformTables &t) {
  OutTables o{};
  for (int r = 0; r < kTransformSeeds; ++r)
    for (int e = 0; e < 64; ++e) {
      o.perm[r][e] = t.perm[r][e];
      if (t.dl[r][e] < 0) o.dlm[r][e >> 5] |= 1u << (e & 31);
      if (t.dr[r][e] < 0) o.drm[r][e >> 5] |= 1u << (e & 31);
    }
  return o;
}

__device__ __forceinline__ float sflip(float v, uint32_t bit) {
  return __uint_as_float(__float_as_uint(v) ^ (bit << 31));
}

// Lane exchange v[lane ^ h] inside a 16-lane row through DPP: quad
// permutes for h = 1, 2; h = 4 as the half-row mirror (lane ^ 7) then the
// quad reversal (^ 3); h = 8 as the row mirror (^ 15) then the half-row
// mirror (^ 7).  Every lane is written (row and bank masks full).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int H>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (H == 1) return dpp<0xB1>(v);
  else if constexpr (H == 2) return dpp<0x4E>(v);
  else if constexpr (H == 4) return dpp<0x1B>(dpp<0x141>(v));
  else if constexpr (H == 8) return dpp<0x141>(dpp<0x140>(v));
  else return __shfl_xor(v, H);
}

// One butterfly stage over all of a wave's register pairs at once, so the
// exchanges of the 64 registers are in flight together.
template <int H, int FM>
__device__ __forceinline__ void butterfly(float (&F)[FM][2][16], int l32) {
  float p[FM][2][16];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) p[fm][fn][e] = lane_xor<H>(F[fm][fn][e]);
  // the lane with bit h clear keeps self + partner, its partner partner -
  // self: both are partner + (self with its sign flipped on the second lane),
  // the same IEEE sums, one sign-bit XOR and one add (into which the compiler
  // can fold a single DPP move)
  const uint32_t up = (uint32_t)((l32 & H) != 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][fn][e] = p[fm][fn][e] + sflip(F[fm][fn][e], up);
}

// Phi_s (s >= 0) on the 64 outputs of one tile row for every token of the
// wave: element i = 32 fn + l32 of a token is register fn of lane l32 of the
// token's half-wave.  D_R, then H_64 (stages h = 1 .. 16 across lanes, 32
// across the two registers, then 1/8), then P (position i takes element
// perm[i]), then D_L.
template <int FM>
__device__ __forceinline__ void phi_tile(float (&F)[FM][2][16], int s, int lane, uint32_t dr0, uint32_t dr1,
                                         uint32_t dl0, uint32_t dl1, int src0, int src1, bool hi0, bool hi1) {
  const int l32 = lane & 31;
  if (s >= 1) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        F[fm][0][e] = sflip(F[fm][0][e], dr0);
        F[fm][1][e] = sflip(F[fm][1][e], dr1);
      }
  }
  butterfly<1, FM>(F, l32);
  butterfly<2, FM>(F, l32);
  butterfly<4, FM>(F, l32);
  butterfly<8, FM>(F, l32);
  butterfly<16, FM>(F, l32);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float a0 = F[fm][0][e], a1 = F[fm][1][e];
      F[fm][0][e] = (a0 + a1) * 0.125f;
      F[fm][1][e] = (a0 - a1) * 0.125f;
    }
  if (s >= 1) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v0 = __float_as_int(F[fm][0][e]), v1 = __float_as_int(F[fm][1][e]);
        const float w00 = __int_as_float(__builtin_amdgcn_ds_bpermute(src0, v0));
        const float w01 = __int_as_float(__builtin_amdgcn_ds_bpermute(src0, v1));
        const float w10 = __int_as_float(__builtin_amdgcn_ds_bpermute(src1, v0));
        const float w11 = __int_as_float(__builtin_amdgcn_ds_bpermute(src1, v1));
        F[fm][0][e] = sflip(hi0 ? w01 : w00, dl0);
        F[fm][1][e] = sflip(hi1 ? w11 : w10, dl1);
      }
  }
}

// Y~ U on the FM x 32-token slices of F that the wave holds for tile row
// seed s: NaN for a seed outside -1 .. 6, nothing for -1 (the identity).
template <int FM>
__device__ __forceinline__ void out_transform(float (&F)[FM][2][16], int s, int lane, const OutTables &ot) {
  if (s < -1 || s > kTransformSeeds) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][0][e] = F[fm][1][e] = __builtin_nanf("");
    return;
  }
  if (s < 0) return;
  const int l32 = lane & 31;
  uint32_t dl0 = 0, dl1 = 0, dr0 = 0, dr1 = 0;
  int src0 = 0, src1 = 0;
  bool hi0 = false, hi1 = false;
  if (s >= 1) {
    dr0 = (ot.drm[s - 1][0] >> l32) & 1u;
    dr1 = (ot.drm[s - 1][1] >> l32) & 1u;
    dl0 = (ot.dlm[s - 1][0] >> l32) & 1u;
    dl1 = (ot.dlm[s - 1][1] >> l32) & 1u;
    const int j0 = ot.perm[s - 1][l32], j1 = ot.perm[s - 1][32 + l32];
    src0 = 4 * ((lane & 32) | (j0 & 31));
    src1 = 4 * ((lane & 32) | (j1 & 31));
    hi0 = j0 >= 32;
    hi1 = j1 >= 32;
  }
  phi_tile<FM>(F, s, lane, dr0, dr1, dl0, dl1, src0, src1, hi0, hi1);
}

}  // namespace aq
