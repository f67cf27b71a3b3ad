// Long-prefill GEMM of the tile-aligned W4/W8 x A8 linear layer
// (AlignQuant Sec. 3.3 "Prefill weight reuse"; App. E.3 Prefill: for long
// prompts the selected weights of a projection are first prepared as INT8
// tiles in logical tile order, then the matrix-core schedule reuses them
// across activation-row groups; eq. 19 rescale).
//
// Operands:
//   A  = qx, INT8 [M][K] row-major;
//   B  = INT8 tiles in logical order: tile (r, j) at (r*C + j) * 64*b_K bytes,
//        inside a tile b_K/16 panels of [64 rows][16 codes] (the INT8 tile
//        layout of the packed model, so an all-INT8 projection's W8 buffer is
//        already this operand), with FP32 scales [(r*C + j)][64].
//
// Workgroup = WM x WN wavefronts over a (64 WM) x (64 WN) output block; each
// wave owns 64 x 64 outputs as 2 x 2 fragments of v_mfma_i32_32x32x32_i8.
// Per input-tile column j:
//   * both operand slabs move HBM/L2 -> LDS by buffer loads that write LDS
//     directly (no VGPR staging), S stages deep: column j + S - 1 is issued
//     when column j starts; the activation slab's 16-byte chunks are placed
//     XOR-swizzled by (row >> 1), which makes the fragment reads free of LDS
//     bank conflicts, by choosing each lane's global address;
//   * the INT32 accumulators are double-buffered by column parity: the 16
//     MFMAs of column j run while the VALU converts and scales column j-1's
//     products into the FP32 accumulators (eq. 19), so the two pipes overlap
//     inside one wave;
//   * fragments of k-step u+1 are read from LDS while k-step u multiplies.
// The token scale and the bias are applied once at the end.

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_tile_xform.h"

namespace aq {
namespace {

#ifndef AQ_DENSE_WM
#define AQ_DENSE_WM 4
#endif
#ifndef AQ_DENSE_WN
#define AQ_DENSE_WN 2
#endif
#ifndef AQ_DENSE_S
#define AQ_DENSE_S 3
#endif

struct DenseArgs {
  const int8_t *qx;
  const int8_t *E;
  const float *Es;
  const float *sx, *bias;
  float *Y;
  int32_t *P;
  int N, K, R, C, M, MB, NB;
  const int8_t *useeds;  // output transform: per tile row seed (-1 .. 6), or null
  OutTables ot;
  // App. B.3 activation groups (GRP): scales [ceil(M/16)][K/64], group (g, c)
  // at g * kg64 + c; ng16 = ceil(M/16) rows
  const float *sxg;
  int kg64, ng16;
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding): wait until at most n vector-memory
// loads of this wave are outstanding and all LDS/scalar accesses are done.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// GRP: the pages' activation groups (App. B.3): one activation scale per 16
// token rows x 64 features, so a 128-column tile's product splits into two
// 64-feature halves (k-steps 0-1 and 2-3), each rescaled with the product of
// its activation scale and the row's weight scale (eq. 19 per group).
template <int BK, int WM, int WN, int S, bool PARTIALS, bool XFORM, bool GRP>
__global__ __launch_bounds__(64 * WM * WN, 1) void prefill_dense_kernel(const DenseArgs a) {
  static_assert(!GRP || (BK == 128 && !XFORM), "grouped activations: b_K = 128, no output transform");
  constexpr int NW = WM * WN;
  constexpr int BM = 64 * WM, BN = 64 * WN;
  constexpr int NP = BK / 16;        // 16-byte chunks per row of a column; panels per tile
  constexpr int KS = BK / 32;        // MFMA k-steps per column
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  constexpr int A_PW = A_BYTES / 1024 / NW;  // 1 KB DMA instructions per wave per column
  constexpr int B_PW = B_BYTES / 1024 / NW;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "even DMA split");
  static_assert(S >= 2 && S <= 4, "stages");
  constexpr int PER_COL = A_PW + B_PW + 1 + (GRP ? 1 : 0);  // VMEM loads a wave issues per column
  static_assert((S - 2) * PER_COL <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) int8_t As0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t As1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t As2[S > 2 ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) int8_t As3[S > 3 ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) int8_t Bs0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t Bs1[B_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t Bs2[S > 2 ? B_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) int8_t Bs3[S > 3 ? B_BYTES : 16];
  // per-wave scale slots: the 64 row scales of the wave's tile, per stage
  __shared__ __attribute__((aligned(1024))) float Ss0[NW * 64];
  __shared__ __attribute__((aligned(1024))) float Ss1[NW * 64];
  __shared__ __attribute__((aligned(1024))) float Ss2[S > 2 ? NW * 64 : 4];
  __shared__ __attribute__((aligned(1024))) float Ss3[S > 3 ? NW * 64 : 4];
  // GRP: per-wave slots of the column's activation-group scales (8 used)
  __shared__ __attribute__((aligned(256))) float Xg0[GRP ? NW * 64 : 4];
  __shared__ __attribute__((aligned(256))) float Xg1[GRP ? NW * 64 : 4];
  __shared__ __attribute__((aligned(256))) float Xg2[GRP && S > 2 ? NW * 64 : 4];
  __shared__ __attribute__((aligned(256))) float Xg3[GRP && S > 3 ? NW * 64 : 4];

  // Rasterization: hardware places block k on XCD k % 8; logical block
  // L = (k % 8) * (G / 8) + k / 8 gives each XCD a contiguous range, walked
  // GROUP_M M-blocks down one N-block column at a time, so the blocks an XCD
  // holds at once share A and B slices in its L2.
  constexpr int GROUP_M = 8;
  const int G = gridDim.x;
  const int kb = blockIdx.x;
  const int per = G / 8;
  const int L = (kb < per * 8) ? (kb % 8) * per + kb / 8 : kb;
  const int in_group = GROUP_M * a.NB;
  const int first_m = (L / in_group) * GROUP_M;
  const int gsize = min(a.MB - first_m, GROUP_M);
  const int bm = first_m + (L % in_group) % gsize;
  const int bn = (L % in_group) / gsize;
  const int m0 = bm * BM;
  const int r0 = WN * bn;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int rw = r0 + wn;
  const int h = lane >> 5;

  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.qx, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rE =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.E, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rS =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.Es, 0, 0x7FFFFFFF, 0x00020000);

  // ---- per-lane DMA source offsets (fixed over j; the column enters as the
  // scalar offset).  A: LDS chunk c = (wave*A_PW + i)*64 + lane of the slab is
  // row c / NP, physical chunk c % NP, which holds logical chunk
  // (c % NP) ^ ((row >> 1) & (NP - 1)).  Rows past M read row M - 1.
  auto a_off = [&](int i, int ln) -> uint32_t {
    const int c = (wave * A_PW + i) * 64 + ln;
    const int row = c / NP, pp = c % NP;
    const int p = pp ^ ((row >> 1) & (NP - 1));
    return (uint32_t)min(m0 + row, a.M - 1) * (uint32_t)a.K + (uint32_t)p * 16u;
  };
  // B: instruction bi = wave*B_PW + i moves panel bi % NP of tile row
  // r0 + bi / NP; tile rows past R read tile row R - 1.
  auto b_off = [&](int i, int ln) -> uint32_t {
    const int bi = wave * B_PW + i;
    const int r = min(r0 + bi / NP, a.R - 1);
    return ((uint32_t)r * (uint32_t)a.C) * (uint32_t)(64 * BK) + (uint32_t)(bi % NP) * 1024u + (uint32_t)ln * 16u;
  };
  auto s_off = [&](int ln) -> uint32_t {
    return ((uint32_t)min(rw, a.R - 1) * (uint32_t)a.C * 64u + (uint32_t)ln) * 4u;
  };
  uint32_t a_voff[A_PW], b_voff[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) a_voff[i] = a_off(i, lane);
#pragma unroll
  for (int i = 0; i < B_PW; ++i) b_voff[i] = b_off(i, lane);
  const uint32_t s_voff = s_off(lane);

  // ---- per-lane fragment read offsets inside a stage.  Logical chunk
  // p = 2u + h of row `row` sits at physical chunk p ^ sw(row); since 2u and h
  // occupy different bits, its offset is af0 ^ (32 u) with af0 the k-step 0
  // offset (row * b_K leaves bits 4-6 clear).  B panels are 1 KB apart, so
  // k-step u adds 2048 u.
  int af0[2], bf0[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int row = wm * 64 + f * 32 + (lane & 31);
    af0[f] = row * BK + ((h ^ ((row >> 1) & (NP - 1))) * 16);
    bf0[f] = (wn * NP + h) * 1024 + (f * 32 + (lane & 31)) * 16;
  }

  auto stageA = [&](int s) -> int8_t * {
    return s == 0 ? As0 : s == 1 ? As1 : s == 2 ? As2 : As3;
  };
  auto stageB = [&](int s) -> int8_t * {
    return s == 0 ? Bs0 : s == 1 ? Bs1 : s == 2 ? Bs2 : Bs3;
  };
  auto stageS = [&](int s) -> float * {
    return (s == 0 ? Ss0 : s == 1 ? Ss1 : s == 2 ? Ss2 : Ss3) + wave * 64;
  };

  float scp0 = 0.f, scp1 = 0.f;  // scales of the column being rescaled
  float scn0 = 0.f, scn1 = 0.f;  // scales of the column being multiplied
  // GRP: activation-group scales of the wave's four 16-row groups (rows
  // m0 + wm*64 + 16 q, q = 2 fm + half), for the two 64-feature groups of the
  // column being multiplied (xc) and the second group's of the previous
  // column (xp); wave-uniform, kept in scalar registers.  They arrive with
  // the column's other loads: lane l of a wave moves the scale of row group
  // (l >> 1) & 3, feature group l & 1 into the wave's slot.
  float xp[4] = {};
  const __amdgpu_buffer_rsrc_t rX =
      __builtin_amdgcn_make_buffer_rsrc((void *)(GRP && a.sxg ? (const void *)a.sxg : (const void *)a.qx), 0,
                                        0x7FFFFFFF, 0x00020000);
  const uint32_t x_voff = GRP && a.sxg
                              ? ((uint32_t)min((m0 + wm * 64) / 16 + ((lane >> 1) & 3), a.ng16 - 1) *
                                     (uint32_t)a.kg64 + (uint32_t)(lane & 1)) * 4u
                              : 0u;
  auto stageX = [&](int s) -> float * {
    return (s == 0 ? Xg0 : s == 1 ? Xg1 : s == 2 ? Xg2 : Xg3) + wave * 64;
  };

  // issue the loads of column j into stage s
  auto issue = [&](int j, int s) {
    int8_t *As_ = stageA(s);
    int8_t *Bs_ = stageB(s);
#pragma unroll
    for (int i = 0; i < A_PW; ++i)
      dma16(rq, As_ + (wave * A_PW + i) * 1024, a_voff[i], (uint32_t)j * BK);
#pragma unroll
    for (int i = 0; i < B_PW; ++i)
      dma16(rE, Bs_ + (wave * B_PW + i) * 1024, b_voff[i], (uint32_t)j * (64 * BK));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)stageS(s), 4, s_voff, (uint32_t)j * 256u, 0, 0);
    if constexpr (GRP)  // (the debug products pass no scales: a harmless read of qx)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_ptr_t)stageX(s), 4, x_voff, a.sxg ? (uint32_t)j * 8u : 0u,
                                               0, 0);
  };

  float F[2][2][16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][fn][e] = 0.f;
  v16i acc[2][2][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) acc[b][fm][fn] = v16i{0};

  // Every column issues exactly one batch of loads, unconditionally (a
  // column index past the end reloads column C - 1 into a stage that is never
  // read), so the wait count below is the same for every column and the
  // compiler sees no conditional LDS writes.  The loop body is unrolled U
  // times so that stage (j % S) and accumulator parity (j % 2) are
  // compile-time; whole groups of U columns run unguarded, then the tail.
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(min(s, a.C - 1), s);

  constexpr int U = (S % 2 == 0) ? S : 2 * S;
  auto column = [&](const int q, const int j) {
    const int s = q % S;
    const int par = q & 1;
    // column j's loads, issued S-1 columns ago, are complete in this wave;
    // after the barrier, in every wave, and stage (j-1) % S is free
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((S - 2) * PER_COL));
    __builtin_amdgcn_s_barrier();
    if constexpr (GRP && !PARTIALS) {
      // the previous column's second-group scales, from its stage slot
      // before the issue below refills that stage.  Column 0 has none: its
      // slot has not been loaded (it holds what an earlier kernel left in
      // LDS, possibly a NaN, which times the zero products would still be
      // NaN), so its scales are zero.
      const float *xs_ = stageX((q + S - 1) % S);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xp[i] = j > 0 ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(xs_[2 * i + 1]))) : 0.f;
    }
    issue(min(j + S - 1, a.C - 1), (q + S - 1) % S);
    scp0 = scn0;
    scp1 = scn1;
    scn0 = stageS(s)[lane & 31];
    scn1 = stageS(s)[32 + (lane & 31)];
    // GRP: the activation-group scales of the previous column's second group
    // (rescaled during k-steps 0-1) and of this column's (first group during
    // k-steps 2-3, second after the column)

    const int8_t *As_ = stageA(s);
    const int8_t *Bs_ = stageB(s);
    v4i fa[2][2], fb[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      fa[0][f] = *reinterpret_cast<const v4i *>(As_ + af0[f]);
      fb[0][f] = *reinterpret_cast<const v4i *>(Bs_ + bf0[f]);
    }
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int cb = u & 1, nb = cb ^ 1;
      if (u + 1 < KS) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          fa[nb][f] = *reinterpret_cast<const v4i *>(As_ + (af0[f] ^ (32 * (u + 1))));
          fb[nb][f] = *reinterpret_cast<const v4i *>(Bs_ + bf0[f] + (u + 1) * 2048);
        }
      }
      if constexpr (GRP) {
        // k-steps 0-1: the first 64-feature group into set 0; 2-3: the second
        // into set 1.  Set 1 holds the previous column's second group until
        // its rescale (k-steps 0-1) is done; set 0 is rescaled in k-steps 2-3.
        const int hs = u >> 1;
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
            acc[hs][fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                fa[cb][fm], fb[cb][fn], (u & 1) == 0 ? v16i{0} : acc[hs][fm][fn], 0, 0, 0);
        if constexpr (!PARTIALS) {
          // this k-step rescales fragment row fm = u & 1 of the other set;
          // its two 16-row groups (rows 8 (e / 4) + 4 h + (e & 3): e >= 8 is
          // the second) take the products of their activation scale and the
          // row's weight scale
          const int fm = u & 1;
          float pr[2][2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const float x = hs == 0 ? xp[2 * fm + hf]
                                    : __int_as_float(__builtin_amdgcn_readfirstlane(
                                          __float_as_int(stageX(s)[2 * (2 * fm + hf)])));
            pr[hf][0] = x * (hs == 0 ? scp0 : scn0);
            pr[hf][1] = x * (hs == 0 ? scp1 : scn1);
          }
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              F[fm][fn][e] = fmaf((float)acc[hs ^ 1][fm][fn][e], pr[e >= 8][fn], F[fm][fn][e]);
        }
        continue;
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[par][fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              fa[cb][fm], fb[cb][fn], u == 0 ? v16i{0} : acc[par][fm][fn], 0, 0, 0);
      if constexpr (!PARTIALS) {
        // rescale 4 / KS fragments of the previous column per k-step
#pragma unroll
        for (int g = 0; g < 4 / KS; ++g) {
          const int fi = u * (4 / KS) + g;
          const int fm = fi >> 1, fn = fi & 1;
          const float scv = fn ? scp1 : scp0;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            F[fm][fn][e] = fmaf((float)acc[par ^ 1][fm][fn][e], scv, F[fm][fn][e]);
        }
      }
    }
    if constexpr (!PARTIALS) {
      // Issue order of the column: the loads of column j + S - 1, the scale
      // and k-step 0 fragment reads, VALU rescale work while those reads are
      // in flight, then per MFMA a slice of the rescale and one fragment read
      // of the next k-step, so that the MFMA and VALU pipes overlap.
      // (GRP: twice the rescale work, 16 VALU per MFMA, plus the scale products)
      constexpr int VPM = GRP ? (256 - 16) / (4 * KS) : (128 - 16) / (4 * KS);
      __builtin_amdgcn_sched_group_barrier(0x020, A_PW + B_PW + 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, GRP ? 32 : 16, 0);
#pragma unroll
      for (int u = 0; u < KS; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          if (u + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    if constexpr (PARTIALS) {
      // 32x32 MFMA result: column (output n) = lane & 31, row (token) =
      // 8 (e / 4) + 4 (lane >> 5) + (e & 3).  GRP: the two 64-feature groups'
      // products, P[m][n][2 j + g].
      if (rw < a.R) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int m = m0 + wm * 64 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3);
              const size_t n = (size_t)rw * 64 + fn * 32 + (lane & 31);
              if (m < a.M) {
                if constexpr (GRP) {
                  a.P[((size_t)m * a.N + n) * a.kg64 + 2 * j] = acc[0][fm][fn][e];
                  a.P[((size_t)m * a.N + n) * a.kg64 + 2 * j + 1] = acc[1][fm][fn][e];
                } else {
                  a.P[((size_t)m * a.N + n) * a.C + j] = acc[par][fm][fn][e];
                }
              }
            }
      }
    }
  };

  int j0 = 0;
  for (; j0 + U <= a.C; j0 += U) {
#pragma unroll
    for (int q = 0; q < U; ++q) column(q, j0 + q);
  }
#pragma unroll
  for (int q = 0; q < U - 1; ++q)
    if (j0 + q < a.C) column(q, j0 + q);
  // no load into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

  if constexpr (!PARTIALS) {
    // the last column's products
    const int lastpar = ((a.C - 1) % U) & 1;  // parity of column C - 1
    const float l0 = scn0, l1 = scn1;
    if constexpr (GRP) {
      // the last column's second 64-feature group (set 1); its stage is
      // (C - 1) % S, never refilled past the end
      const float *xs_ = stageX((a.C - 1) % S);
      float xl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xl[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(xs_[2 * i + 1])));
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = xl[2 * fm + (e >= 8)];
          F[fm][0][e] = fmaf((float)acc[1][fm][0][e], x * l0, F[fm][0][e]);
          F[fm][1][e] = fmaf((float)acc[1][fm][1][e], x * l1, F[fm][1][e]);
        }
    } else if (lastpar == 0) {
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          F[fm][0][e] = fmaf((float)acc[0][fm][0][e], l0, F[fm][0][e]);
          F[fm][1][e] = fmaf((float)acc[0][fm][1][e], l1, F[fm][1][e]);
        }
    } else {
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          F[fm][0][e] = fmaf((float)acc[1][fm][0][e], l0, F[fm][0][e]);
          F[fm][1][e] = fmaf((float)acc[1][fm][1][e], l1, F[fm][1][e]);
        }
    }
    if (rw >= a.R) return;
    if constexpr (XFORM) {
      // Y = Y~ U on this wave's tile row (the 64 outputs of a token sit in
      // one half-wave), before the token scale and the bias
      out_transform<2>(F, a.useeds[rw], lane, a.ot);
    }
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3);
        if (m >= a.M) continue;
        const float sxm = GRP ? 1.0f : a.sx[m];  // GRP: the group scales are in F already
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          const size_t n = (size_t)rw * 64 + fn * 32 + (lane & 31);
          float v = GRP ? F[fm][fn][e] : F[fm][fn][e] * sxm;
          if (a.bias) v += a.bias[n];
          // non-temporal: the outputs are not read again here, and keeping them
          // out of the caches leaves room for the operand slabs other blocks re-read
          __builtin_nontemporal_store(v, a.Y + (size_t)m * a.N + n);
        }
      }
  }
}

template <int BK, int WM, int WN, int S>
hipError_t launch_dense_cfg(const DenseArgs &args, bool partials, hipStream_t stream) {
  const dim3 grid(args.MB * args.NB), block(64 * WM * WN);
  if (partials)
    hipLaunchKernelGGL((prefill_dense_kernel<BK, WM, WN, S, true, false, false>), grid, block, 0, stream, args);
  else if (args.useeds)
    hipLaunchKernelGGL((prefill_dense_kernel<BK, WM, WN, S, false, true, false>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((prefill_dense_kernel<BK, WM, WN, S, false, false, false>), grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_dense(const int8_t *E, const float *Es, int N, int K, int bK,
                                const int8_t *qx, const float *sx, int M, const float *bias,
                                float *Y, int32_t *P, hipStream_t stream, const int8_t *useeds,
                                const TransformTables *tables) {
  constexpr int WM = AQ_DENSE_WM, WN = AQ_DENSE_WN, S = AQ_DENSE_S;
  DenseArgs args;
  args.useeds = useeds;
  args.ot = useeds && tables ? out_tables(*tables) : OutTables{};
  args.qx = qx; args.E = E; args.Es = Es; args.sx = sx; args.bias = bias; args.Y = Y; args.P = P;
  args.N = N; args.K = K; args.R = N / 64; args.C = K / bK; args.M = M;
  args.MB = (M + 64 * WM - 1) / (64 * WM);
  args.NB = (args.R + WN - 1) / WN;
  if (bK == 128) return launch_dense_cfg<128, WM, WN, S>(args, P != nullptr, stream);
  return launch_dense_cfg<64, WM, WN, S>(args, P != nullptr, stream);
}

hipError_t launch_prefill_dense_grouped(const int8_t *E, const float *Es, int N, int K, const int8_t *qx,
                                        const float *sxg, int M, const float *bias, float *Y, int32_t *P,
                                        hipStream_t stream) {
  constexpr int WM = AQ_DENSE_WM, WN = AQ_DENSE_WN, S = AQ_DENSE_S;
  DenseArgs args{};
  args.qx = qx; args.E = E; args.Es = Es; args.sx = nullptr; args.bias = bias; args.Y = Y; args.P = P;
  args.N = N; args.K = K; args.R = N / 64; args.C = K / 128; args.M = M;
  args.MB = (M + 64 * WM - 1) / (64 * WM);
  args.NB = (args.R + WN - 1) / WN;
  args.useeds = nullptr;
  args.sxg = sxg;
  args.kg64 = K / 64;
  args.ng16 = (M + 15) / 16;
  const dim3 grid(args.MB * args.NB), block(64 * WM * WN);
  if (P)
    hipLaunchKernelGGL((prefill_dense_kernel<128, WM, WN, S, true, false, true>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((prefill_dense_kernel<128, WM, WN, S, false, false, true>), grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace aq
