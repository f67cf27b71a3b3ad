// Tile-aligned orthogonal transforms (AlignQuant App. B.1, eq. 4).
//
// Phi_-1 = I, Phi_0 = H_64 (normalized Hadamard, entries +-1/8), and
// Phi_s = D_L,s P_s H_64 D_R,s for s = 1 .. 6, the signed permutations given
// by the caller ((P v)_i = v[perm[i]]).  V = diag(Phi_{v_c}) acts on the
// 64-feature blocks of activation and weight rows (X~ = X V, W V), U_r =
// Phi_{u_r}^T on the 64 rows of output tile row r (W~ = U W V), and the
// output returns by Y = Y~ U.
//
// One wavefront transforms one 64-element block, lane l holding element l:
// the signs are per-lane multiplies, the permutation one cross-lane move
// (ds_permute pushes for P^T, ds_bpermute pulls for P), H_64 six butterfly
// stages over lane pairs l, l ^ h in the order h = 1, 2, .., 32 (the lane
// with bit h clear keeps a + b, its partner a - b), then the exact 1/8.
// Every value that later feeds a quantizer (X~, W~) is produced by exactly
// that FP32 sequence.
//
// Two lane layouts compute that same sequence:
//  - one block per wavefront, lane l holding element l (the butterflies are
//    cross-lane shuffles): the offline weight transform, which also needs the
//    column pass;
//  - the quad layout of the online activation and output transforms: a
//    wavefront takes 16 blocks, the 4 lanes of quad b hold block b, lane q
//    its elements 16q .. 16q+15 (64 contiguous bytes, four 16-byte loads).
//    Stages h = 1 .. 8 pair registers of one lane; h = 16 and 32 pair lanes
//    q ^ 1 and q ^ 2 of the quad, through DPP quad permutes (full-rate
//    vector ALU, no LDS round trip); the permutation goes through LDS, a
//    scatter and a contiguous read (or the reverse).
// The signed permutations travel in the kernel arguments: the tables as the
// caller gives them (one-block layout) and, for the quad layout, rows r =
// s + 1 for s = -1 .. 6 (rows 0 and 1 the identity) with the signs as bit
// masks, copied to LDS at entry.  Seeds are read from device memory.

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_quant.h"

namespace aq {
namespace {

// Tables of the quad layout: row r = s + 1 (s = -1 .. 6), perm bytes and
// sign masks (bit e set: element e negated).
constexpr int kQuadRows = kTransformSeeds + 2;
struct QuadTables {
  uint8_t perm[kQuadRows][64];
  uint64_t dlm[kQuadRows], drm[kQuadRows];
};
// the longest row the one-pass quantizer stages, plus its tables and the
// reduction slots of 16 waves, fit the 160 KiB of LDS
static_assert((size_t)kQuantTransformMaxK * 4 + sizeof(QuadTables) + 16 * 4 <= 160 * 1024,
              "one-pass row staging exceeds LDS");

// Lane l's entries of the six tables.
struct LaneTab {
  int perm[kTransformSeeds];
  float dl[kTransformSeeds], dr[kTransformSeeds];
};

__device__ __forceinline__ LaneTab lane_tab(const TransformTables &t, int lane) {
  LaneTab r;
#pragma unroll
  for (int j = 0; j < kTransformSeeds; ++j) {
    r.perm[j] = t.perm[j][lane];
    r.dl[j] = (float)t.dl[j][lane];
    r.dr[j] = (float)t.dr[j][lane];
  }
  return r;
}

// Entries of seed s >= 1 (s wave-uniform: a chain of selects).
struct Signed {
  int perm;
  float dl, dr;
};
__device__ __forceinline__ Signed pick(const LaneTab &t, int s) {
  Signed r{0, 1.f, 1.f};
#pragma unroll
  for (int j = 0; j < kTransformSeeds; ++j)
    if (s == j + 1) r = Signed{t.perm[j], t.dl[j], t.dr[j]};
  return r;
}

__device__ __forceinline__ bool seed_ok(int s) { return s >= -1 && s <= kTransformSeeds; }

// H_64 v over the wave, then the exact scaling by 1/8.
__device__ __forceinline__ float fwht64(float v, int lane) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float p = __shfl_xor(v, h);
    v = (lane & h) ? p - v : v + p;
  }
  return v * 0.125f;
}

// Phi_s^T v = D_R H P^T D_L v; NaN for a seed outside -1 .. 6.
__device__ __forceinline__ float phi_t(float v, int s, int lane, const LaneTab &t) {
  if (!seed_ok(s)) return __builtin_nanf("");
  if (s < 0) return v;
  if (s == 0) return fwht64(v, lane);
  const Signed e = pick(t, s);
  // P^T: element i moves to position perm[i]
  const float w = __int_as_float(__builtin_amdgcn_ds_permute(4 * e.perm, __float_as_int(v * e.dl)));
  return fwht64(w, lane) * e.dr;
}

// Phi_s v = D_L P H D_R v; NaN for a seed outside -1 .. 6.
__device__ __forceinline__ float phi(float v, int s, int lane, const LaneTab &t) {
  if (!seed_ok(s)) return __builtin_nanf("");
  if (s < 0) return v;
  if (s == 0) return fwht64(v, lane);
  const Signed e = pick(t, s);
  const float h = fwht64(v * e.dr, lane);
  // P: position i takes element perm[i]
  return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * e.perm, __float_as_int(h))) * e.dl;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---- quad layout

__device__ __forceinline__ void copy_quad_tables(QuadTables &dst, const QuadTables &src) {
  constexpr int kWords = sizeof(QuadTables) / 4;
  for (int i = threadIdx.x; i < kWords; i += blockDim.x)
    reinterpret_cast<uint32_t *>(&dst)[i] = reinterpret_cast<const uint32_t *>(&src)[i];
}

// A lane's part of its block's transform: the permutation entries of its 16
// elements (byte k of perm = entry of element 16q + k), the sign bits of
// D_L and D_R (bit k: element 16q + k negated), identity, invalid seed.
struct QuadEntry {
  uint4 perm;
  uint32_t dl, dr;
  bool ident, bad;
};

__device__ __forceinline__ QuadEntry quad_entry(const QuadTables &st, int s, int q) {
  QuadEntry e;
  e.bad = !seed_ok(s);
  e.ident = s == -1;
  const int r = e.bad ? 0 : s + 1;
  e.perm = *reinterpret_cast<const uint4 *>(&st.perm[r][16 * q]);
  e.dl = (uint32_t)(st.dlm[r] >> (16 * q)) & 0xFFFFu;
  e.dr = (uint32_t)(st.drm[r] >> (16 * q)) & 0xFFFFu;
  return e;
}

__device__ __forceinline__ int perm_at(const uint4 &p, int k) {
  const uint32_t w = k < 4 ? p.x : k < 8 ? p.y : k < 12 ? p.z : p.w;
  return (int)((w >> (8 * (k & 3))) & 0xFFu);
}

// Multiplication by +-1, exactly: the sign bit flipped where bit k is set.
__device__ __forceinline__ float flip(float v, uint32_t bits, int k) {
  return __uint_as_float(__float_as_uint(v) ^ (((bits >> k) & 1u) << 31));
}

template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// H_64 over the quad's block, in the order h = 1, 2, .., 32, then 1/8.
__device__ __forceinline__ void fwht_quad(float (&r)[16], int q) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (!(k & h)) {
        const float a = r[k], b = r[k + h];
        r[k] = a + b;
        r[k + h] = a - b;
      }
  // h = 16 and 32 pair lanes q, q ^ 1 and q, q ^ 2.  The lane with the
  // bit clear keeps self + partner, its partner partner - self: both are
  // partner + (self with its sign flipped on the second lane), the same
  // IEEE sums, one sign-bit XOR and one add (the DPP move folds into it).
  const uint32_t f16 = (uint32_t)(q & 1) << 31, f32 = (uint32_t)((q >> 1) & 1) << 31;
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = quad_xor<0xB1>(r[k]) + __uint_as_float(__float_as_uint(r[k]) ^ f16);
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = quad_xor<0x4E>(r[k]) + __uint_as_float(__float_as_uint(r[k]) ^ f32);
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] *= 0.125f;
}

// This wave's LDS accesses complete, in order, before the next ones.
__device__ __forceinline__ void wave_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Phi_s^T = D_R H P^T D_L on the quad's block; wl: the block's 64 floats of
// LDS (used only when ok; every lane of the wave calls this).
__device__ __forceinline__ void quad_phi_t(float (&r)[16], const QuadEntry &e, int q, float *wl, bool ok) {
  if (ok) {
#pragma unroll
    for (int k = 0; k < 16; ++k) wl[perm_at(e.perm, k)] = flip(r[k], e.dl, k);  // P^T: to perm[i]
  }
  wave_lds_wait();
  if (ok) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const float4 w = reinterpret_cast<const float4 *>(wl)[4 * q + k4];
      r[4 * k4] = w.x; r[4 * k4 + 1] = w.y; r[4 * k4 + 2] = w.z; r[4 * k4 + 3] = w.w;
    }
  }
  wave_lds_wait();
  float h[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) h[k] = r[k];
  fwht_quad(h, q);
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = e.bad ? __builtin_nanf("") : flip(e.ident ? r[k] : h[k], e.dr, k);
}

// Phi_s = D_L P H D_R on the quad's block.
__device__ __forceinline__ void quad_phi(float (&r)[16], const QuadEntry &e, int q, float *wl, bool ok) {
  float h[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) h[k] = r[k] = flip(r[k], e.dr, k);
  fwht_quad(h, q);
  if (ok) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int k = 4 * k4;
      reinterpret_cast<float4 *>(wl)[4 * q + k4] =
          e.ident ? make_float4(r[k], r[k + 1], r[k + 2], r[k + 3]) : make_float4(h[k], h[k + 1], h[k + 2], h[k + 3]);
    }
  }
  wave_lds_wait();
  if (ok) {
#pragma unroll
    for (int k = 0; k < 16; ++k) r[k] = wl[perm_at(e.perm, k)];  // P: from perm[i]
  }
  wave_lds_wait();
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = e.bad ? __builtin_nanf("") : flip(r[k], e.dl, k);
}

__device__ __forceinline__ void load16(float (&r)[16], const float *p, bool ok) {
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const float4 v = ok ? reinterpret_cast<const float4 *>(p)[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
    r[4 * k4] = v.x; r[4 * k4 + 1] = v.y; r[4 * k4 + 2] = v.z; r[4 * k4 + 3] = v.w;
  }
}

struct TransformArgs {
  const float *src;
  float *dst;
  int rows, cols;          // matrix [rows][cols], cols a multiple of 64
  const int8_t *seeds;     // per 64-feature block of a row (cols / 64)
  const int8_t *seeds2;    // weights only: per 64-row tile row (rows / 64)
  const float *bias;       // output transform only: added after it, or null
  TransformTables t;
  QuadTables qt;
};

// Rows, quad layout: workgroup (x, y) covers blocks 64 y .. 64 y + 63 of
// row x, 16 per wave.  FORWARD: Phi^T per block (X V); otherwise Phi per
// block (Y~ U) plus the bias.  src == dst is allowed: each lane reads its
// 16 elements before it writes them.
template <bool FORWARD>
__global__ __launch_bounds__(256) void transform_rows_kernel(const TransformArgs a) {
  __shared__ QuadTables st;
  __shared__ float4 buf[4][16 * 16];  // per wave: 16 blocks of 64 floats
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int b = lane >> 2, q = lane & 3;
  const int nb = a.cols / 64;
  const int c = blockIdx.y * 64 + wave * 16 + b;
  const bool ok = c < nb;
  const size_t off = (size_t)blockIdx.x * a.cols + (size_t)c * 64 + 16 * q;
  const int s = ok ? (int)a.seeds[c] : -1;
  float r[16];
  load16(r, a.src + off, ok);
  copy_quad_tables(st, a.qt);
  __syncthreads();
  const QuadEntry e = quad_entry(st, s, q);
  float *wl = reinterpret_cast<float *>(&buf[wave][16 * b]);
  if (FORWARD) {
    quad_phi_t(r, e, q, wl, ok);
  } else {
    quad_phi(r, e, q, wl, ok);
    if (a.bias && ok) {
      float bb[16];
      load16(bb, a.bias + (size_t)c * 64 + 16 * q, true);
#pragma unroll
      for (int k = 0; k < 16; ++k) r[k] += bb[k];
    }
  }
  if (ok) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      reinterpret_cast<float4 *>(a.dst + off)[k4] = make_float4(r[4 * k4], r[4 * k4 + 1], r[4 * k4 + 2], r[4 * k4 + 3]);
  }
}

// W~ = U W V for one 64 x 64 block (tile row r, column block c): the rows
// by Phi_{v_c}^T, then the columns by U_r = Phi_{u_r}^T, staged in LDS
// (row pitch 65 words: column reads hit 64 distinct banks).
__global__ __launch_bounds__(256) void transform_weights_kernel(const TransformArgs a) {
  __shared__ float blk[64][65];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c = blockIdx.x, r = blockIdx.y;
  const int sv = a.seeds[c], su = a.seeds2[r];
  const LaneTab tab = lane_tab(a.t, lane);
  const float *src = a.src + (size_t)r * 64 * a.cols + (size_t)c * 64;
  for (int i = wave; i < 64; i += 4) blk[i][lane] = phi_t(src[(size_t)i * a.cols + lane], sv, lane, tab);
  __syncthreads();
  // each wave transforms, in place, the columns k = wave (mod 4)
  for (int k = wave; k < 64; k += 4) blk[lane][k] = phi_t(blk[lane][k], su, lane, tab);
  __syncthreads();
  float *dst = a.dst + (size_t)r * 64 * a.cols + (size_t)c * 64;
  for (int i = wave; i < 64; i += 4) dst[(size_t)i * a.cols + lane] = blk[i][lane];
}

// X V followed by the per-token quantizer of App. B.3 in one pass: one
// workgroup per token row; the waves transform the row's 64-blocks into LDS
// (FP32, the order above) while reducing max |x~|, then every thread writes
// the codes of its float4 groups.  The transformed row never leaves the chip.
struct QuantTArgs {
  const float *X;
  int K;
  const int8_t *seeds;
  int8_t *qx;
  float *sx;
  QuadTables qt;
};

template <int T>
__global__ __launch_bounds__(T) void quant_act_transformed_kernel(const QuantTArgs a) {
  extern __shared__ float4 xt4[];  // the transformed row, K floats
  __shared__ QuadTables st;
  float *xt = reinterpret_cast<float *>(xt4);
  constexpr int W = T / 64;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int b = lane >> 2, q = lane & 3;
  const int nb = a.K >> 6;
  const size_t m = blockIdx.x;
  const float *row = a.X + m * a.K;
  // the first group's loads are in flight while the tables are copied
  int g = wave, c = 16 * g + b;
  bool ok = c < nb;
  int s = ok ? (int)a.seeds[c] : -1;
  float r[16];
  load16(r, row + (size_t)c * 64 + 16 * q, ok);
  copy_quad_tables(st, a.qt);
  __syncthreads();
  uint32_t amax = 0;
  while (16 * g < nb) {  // wave-uniform
    const QuadEntry e = quad_entry(st, s, q);
    // the block's own slots in the row serve as the permutation's staging
    quad_phi_t(r, e, q, xt + (size_t)(ok ? c : 0) * 64, ok);
    if (ok) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int k = 4 * k4;
        xt4[c * 16 + 4 * q + k4] = make_float4(r[k], r[k + 1], r[k + 2], r[k + 3]);
        amax = max(amax, max(max(abs_bits(r[k]), abs_bits(r[k + 1])), max(abs_bits(r[k + 2]), abs_bits(r[k + 3]))));
      }
    }
    g += W;
    c = 16 * g + b;
    ok = c < nb;
    if (16 * g < nb) {
      s = ok ? (int)a.seeds[c] : -1;
      load16(r, row + (size_t)c * 64 + 16 * q, ok);
    }
  }
  // its barrier also publishes xt; a NaN (a seed outside -1 .. 6) makes the
  // scale NaN rather than the 1e-12 floor
  const uint32_t am = block_max_u32<T>(amax);
  const double sc = am > 0x7F800000u ? (double)__builtin_nanf("") : row_scale(am);
  if (threadIdx.x == 0) a.sx[m] = (float)sc;
  const float inv = (float)(1.0 / sc);
  uint32_t *out = reinterpret_cast<uint32_t *>(a.qx + m * a.K);
  for (int c4 = threadIdx.x; c4 < (a.K >> 2); c4 += T) out[c4] = codes4_fast(xt4[c4], sc, inv);
}

// The one-pass quantizer for few, short rows, lane by element:
// wave w takes blocks w, w + 16, .. of its row, lane l holding element l of
// the block, so that each block is one permute and six butterfly stages of
// cross-lane moves (DPP quad permutes for h = 1, 2, ds_swizzle for h = 4,
// 8, 16, ds_bpermute for h = 32) with no LDS staging of the row.  The same
// FP32 sequence as the quad layout: D_L, then P^T (ds_permute pushes element
// l to position perm[l]), H, the exact 1/8, D_R.
struct LaneTables {
  uint8_t perm[kTransformSeeds][64];
  uint64_t dlm[kTransformSeeds], drm[kTransformSeeds];
};
constexpr int kLaneTabWords = sizeof(LaneTables) / 4;
static_assert(sizeof(LaneTables) % 4 == 0 && kLaneTabWords <= 1024, "lane tables");

struct QuantLArgs {
  const float *X;
  int K;
  const int8_t *seeds;
  int8_t *qx;
  float *sx;
  LaneTables lt;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int PAT>
__device__ __forceinline__ float swz_f(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PAT));
}
// fwht64 with the partners from DPP and ds_swizzle where they reach
__device__ __forceinline__ float fwht64_fast(float v, int lane) {
  float p = dpp_f<0xB1>(v);  // lane ^ 1
  v = (lane & 1) ? p - v : v + p;
  p = dpp_f<0x4E>(v);  // lane ^ 2
  v = (lane & 2) ? p - v : v + p;
  p = swz_f<0x101F>(v);  // lane ^ 4
  v = (lane & 4) ? p - v : v + p;
  p = swz_f<0x201F>(v);  // lane ^ 8
  v = (lane & 8) ? p - v : v + p;
  p = swz_f<0x401F>(v);  // lane ^ 16
  v = (lane & 16) ? p - v : v + p;
  p = __shfl_xor(v, 32);
  v = (lane & 32) ? p - v : v + p;
  return v * 0.125f;
}

template <int NBW>
__global__ __launch_bounds__(1024) void quant_act_transformed_lanes_kernel(const QuantLArgs a) {
  __shared__ LaneTables st;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nb = a.K >> 6;
  const size_t m = blockIdx.x;
  const float *row = a.X + m * a.K;
  float v[NBW];
  int sd[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int c = wave + 16 * j;
    const bool ok = c < nb;  // wave-uniform
    v[j] = ok ? row[(size_t)c * 64 + lane] : 0.f;
    sd[j] = ok ? (int)a.seeds[c] : -1;
  }
  if (threadIdx.x < kLaneTabWords)
    reinterpret_cast<uint32_t *>(&st)[threadIdx.x] = reinterpret_cast<const uint32_t *>(&a.lt)[threadIdx.x];
  __syncthreads();
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    if (wave + 16 * j >= nb) continue;
    const int s = sd[j];
    if (!seed_ok(s)) {
      v[j] = __builtin_nanf("");
    } else if (s >= 0) {
      int dest = lane;
      uint32_t fl = 0u, fr = 0u;
      if (s >= 1) {
        dest = st.perm[s - 1][lane];
        fl = (uint32_t)(st.dlm[s - 1] >> lane) & 1u;
        fr = (uint32_t)(st.drm[s - 1] >> lane) & 1u;
      }
      float x = __uint_as_float(__float_as_uint(v[j]) ^ (fl << 31));                 // D_L
      x = __int_as_float(__builtin_amdgcn_ds_permute(4 * dest, __float_as_int(x)));  // P^T: to perm[l]
      x = fwht64_fast(x, lane);                                                       // H
      v[j] = __uint_as_float(__float_as_uint(x) ^ (fr << 31));                       // D_R
    }
    amax = max(amax, abs_bits(v[j]));
  }
  // a NaN (a seed outside -1 .. 6) makes the scale NaN rather than the floor
  const uint32_t am = block_max_u32<1024>(amax);
  const double sc = am > 0x7F800000u ? (double)__builtin_nanf("") : row_scale(am);
  if (threadIdx.x == 0) a.sx[m] = (float)sc;
  const float inv = (float)(1.0 / sc);
  int8_t *out = a.qx + m * a.K;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int c = wave + 16 * j;
    if (c < nb) out[(size_t)c * 64 + lane] = (int8_t)(code_fast(v[j], sc, inv) & 0xFF);
  }
}

LaneTables lane_tables(const TransformTables &t) {
  LaneTables x{};
  for (int j = 0; j < kTransformSeeds; ++j)
    for (int e = 0; e < 64; ++e) {
      x.perm[j][e] = t.perm[j][e];
      if (t.dl[j][e] < 0) x.dlm[j] |= 1ull << e;
      if (t.dr[j][e] < 0) x.drm[j] |= 1ull << e;
    }
  return x;
}

template <typename Kern, typename Args>
hipError_t launch_lds(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const Args &a) {
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, lds, stream, a);
  return hipGetLastError();
}

QuadTables quad_tables(const TransformTables &t) {
  QuadTables q{};
  for (int r = 0; r < kQuadRows; ++r)
    for (int e = 0; e < 64; ++e) {
      q.perm[r][e] = r < 2 ? (uint8_t)e : t.perm[r - 2][e];
      if (r >= 2 && t.dl[r - 2][e] < 0) q.dlm[r] |= 1ull << e;
      if (r >= 2 && t.dr[r - 2][e] < 0) q.drm[r] |= 1ull << e;
    }
  return q;
}

}  // namespace

hipError_t launch_transform(int kind, const float *src, float *dst, int rows, int cols,
                            const int8_t *seeds, const int8_t *seeds2, const float *bias,
                            const TransformTables &t, hipStream_t stream) {
  TransformArgs a;
  a.src = src;
  a.dst = dst;
  a.rows = rows;
  a.cols = cols;
  a.seeds = seeds;
  a.seeds2 = seeds2;
  a.bias = bias;
  a.t = t;
  a.qt = quad_tables(t);
  const dim3 block(256);
  if (kind == kTransformWeights) {
    hipLaunchKernelGGL(transform_weights_kernel, dim3(cols / 64, rows / 64), block, 0, stream, a);
  } else {
    const dim3 grid(rows, (cols / 64 + 63) / 64);
    if (kind == kTransformRows) hipLaunchKernelGGL(transform_rows_kernel<true>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(transform_rows_kernel<false>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_quant_act_transformed(const float *X, int M, int K, const int8_t *seeds,
                                        const TransformTables &t, int8_t *qx, float *sx,
                                        hipStream_t stream) {
  // few rows of at most 64 blocks: lane by element, the row in registers
  // (measured at M = 1: 3.8-4.0 us against 4.1-4.3 us for the quad layout at
  // K = 3072; at K = 8192, 8 blocks per wave, 7.4 us against 5.9 us)
  const int nb = K / 64;
  if (M < 256 && nb <= 64) {
    QuantLArgs l;
    l.X = X;
    l.K = K;
    l.seeds = seeds;
    l.qx = qx;
    l.sx = sx;
    l.lt = lane_tables(t);
    const dim3 grid(M), block(1024);
    if (nb <= 16) hipLaunchKernelGGL(quant_act_transformed_lanes_kernel<1>, grid, block, 0, stream, l);
    else if (nb <= 32) hipLaunchKernelGGL(quant_act_transformed_lanes_kernel<2>, grid, block, 0, stream, l);
    else hipLaunchKernelGGL(quant_act_transformed_lanes_kernel<4>, grid, block, 0, stream, l);
    return hipGetLastError();
  }
  QuantTArgs a;
  a.X = X;
  a.K = K;
  a.seeds = seeds;
  a.qx = qx;
  a.sx = sx;
  a.qt = quad_tables(t);
  const size_t lds = (size_t)K * sizeof(float);
  // few rows: wide workgroups keep each lane's share short
  if (M < 256) return launch_lds(quant_act_transformed_kernel<1024>, dim3(M), dim3(1024), lds, stream, a);
  return launch_lds(quant_act_transformed_kernel<256>, dim3(M), dim3(256), lds, stream, a);
}

}  // namespace aq
