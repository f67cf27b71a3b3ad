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
// that FP32 sequence.  The six signed permutations travel in the kernel
// arguments (1152 bytes); the per-block seeds are read from device memory.

#include "aq_device.h"
#include "aq_internal.h"

namespace aq {
namespace {

struct TransformArgs {
  const float *src;
  float *dst;
  int rows, cols;          // matrix [rows][cols], cols a multiple of 64
  const int8_t *seeds;     // per 64-feature block of a row (cols / 64)
  const int8_t *seeds2;    // weights only: per 64-row tile row (rows / 64)
  TransformTables t;
};

// H_64 v over the wave, then the exact scaling by 1/8.
__device__ __forceinline__ float fwht64(float v, int lane) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float p = __shfl_xor(v, h);
    v = (lane & h) ? p - v : v + p;
  }
  return v * 0.125f;
}

__device__ __forceinline__ bool seed_ok(int s) { return s >= -1 && s <= kTransformSeeds; }

// Phi_s^T v = D_R H P^T D_L v.
__device__ __forceinline__ float phi_t(float v, int s, int lane, const TransformTables &t) {
  if (s < 0) return v;
  if (s == 0) return fwht64(v, lane);
  const float u = v * (float)t.dl[s - 1][lane];
  // P^T: element i moves to position perm[i]
  const float w = __int_as_float(__builtin_amdgcn_ds_permute(4 * (int)t.perm[s - 1][lane], __float_as_int(u)));
  return fwht64(w, lane) * (float)t.dr[s - 1][lane];
}

// Phi_s v = D_L P H D_R v.
__device__ __forceinline__ float phi(float v, int s, int lane, const TransformTables &t) {
  if (s < 0) return v;
  if (s == 0) return fwht64(v, lane);
  const float h = fwht64(v * (float)t.dr[s - 1][lane], lane);
  // P: position i takes element perm[i]
  const float w = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (int)t.perm[s - 1][lane], __float_as_int(h)));
  return w * (float)t.dl[s - 1][lane];
}

// Row blocks: workgroup (x, y) covers features [1024 y, 1024 y + 1024) of
// row x, each of its 4 waves 4 consecutive 64-blocks (loads first, so 4 are
// in flight).  FORWARD: Phi^T per block (X V); otherwise Phi per block
// (Y~ U).  src == dst is allowed: every element is read before it is
// written, by the same lane.
template <bool FORWARD>
__global__ __launch_bounds__(256) void transform_rows_kernel(const TransformArgs a) {
  const int lane = threadIdx.x & 63;
  const int nb = a.cols / 64;
  const int c0 = blockIdx.y * 16 + (threadIdx.x >> 6) * 4;
  const size_t row = (size_t)blockIdx.x * a.cols;
  float v[4];
  int s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + j;
    s[j] = c < nb ? (int)a.seeds[c] : -1;
    v[j] = c < nb ? a.src[row + (size_t)c * 64 + lane] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + j;
    if (c >= nb) break;  // wave-uniform
    float r = seed_ok(s[j]) ? (FORWARD ? phi_t(v[j], s[j], lane, a.t) : phi(v[j], s[j], lane, a.t))
                            : __builtin_nanf("");
    a.dst[row + (size_t)c * 64 + lane] = r;
  }
}

// W~ = U W V for one 64 x 64 block (tile row r, column block c): the rows
// by Phi_{v_c}^T, then the columns by U_r = Phi_{u_r}^T, staged in LDS
// (row pitch 65 words: column reads hit 64 distinct banks).
__global__ __launch_bounds__(256) void transform_weights_kernel(const TransformArgs a) {
  __shared__ float blk[64][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x, r = blockIdx.y;
  const int sv = a.seeds[c], su = a.seeds2[r];
  const bool ok = seed_ok(sv) && seed_ok(su);
  const float *src = a.src + (size_t)r * 64 * a.cols + (size_t)c * 64;
  for (int i = wave; i < 64; i += 4) blk[i][lane] = phi_t(src[(size_t)i * a.cols + lane], ok ? sv : -1, lane, a.t);
  __syncthreads();
  // each wave transforms, in place, the columns k = wave (mod 4)
  for (int k = wave; k < 64; k += 4) blk[lane][k] = phi_t(blk[lane][k], ok ? su : -1, lane, a.t);
  __syncthreads();
  float *dst = a.dst + (size_t)r * 64 * a.cols + (size_t)c * 64;
  for (int i = wave; i < 64; i += 4) dst[(size_t)i * a.cols + lane] = ok ? blk[i][lane] : __builtin_nanf("");
}

}  // namespace

hipError_t launch_transform(int kind, const float *src, float *dst, int rows, int cols,
                            const int8_t *seeds, const int8_t *seeds2, const TransformTables &t,
                            hipStream_t stream) {
  TransformArgs a;
  a.src = src;
  a.dst = dst;
  a.rows = rows;
  a.cols = cols;
  a.seeds = seeds;
  a.seeds2 = seeds2;
  a.t = t;
  const dim3 block(256);
  if (kind == kTransformWeights) {
    hipLaunchKernelGGL(transform_weights_kernel, dim3(cols / 64, rows / 64), block, 0, stream, a);
  } else {
    const dim3 grid(rows, (cols / 64 + 15) / 16);
    if (kind == kTransformRows) hipLaunchKernelGGL(transform_rows_kernel<true>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(transform_rows_kernel<false>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace aq
