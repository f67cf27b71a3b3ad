// Persistent long-prefill GEMM over 256 x 256 output tiles (AlignQuant Sec. 3.3
// "Prefill weight reuse"; App. E.3 Prefill and eq. 19).
//
// Operands are those of the dense long-prefill route: A = qx INT8 [M][K]; B =
// INT8 tiles in logical order (tile (r, j) at (r*C + j) * 64*128 bytes,
// 8 panels of [64 rows][16 codes]) with FP32 row scales at (r*C + j) * 64.
//
// One workgroup of 8 wavefronts per CU walks its share of the 256 x 256
// output tiles; each tile is C input-tile columns of 128.  The columns of
// all of a workgroup's tiles form one stream:
//   * column g+1's operand slabs (A 32 KB, B 32 KB, the 64 row scales of each
//     wave's tile row, and the tile's token scales and bias) move HBM/L2 ->
//     LDS with buffer loads that write LDS directly while column g
//     multiplies; every column issues the same loads unconditionally (a
//     column past the end reloads the last one), so the only waits on them
//     are the explicit ones at the column boundary;
//   * a wave owns 128 x 64 outputs (FP32 accumulators in registers) and walks
//     them as four 32 x 64 sub-tiles per column, 8 MFMAs each
//     (v_mfma_i32_32x32x32_i8); the INT32 products alternate between two
//     register sets, so each sub-tile's eq. 19 rescale (convert, multiply by
//     the tile's per-row scale, add) runs on the VALU under the next
//     sub-tile's MFMAs; the weight fragments of a column stay in registers
//     across its four sub-tiles;
//   * a finished tile's outputs (x token scale, + bias) are stored at the
//     start of the next tile's first column, so the stores drain while that
//     column multiplies.
// 256 x 256 tiles halve the operand bytes per multiply-add of 128 x 128
// tiles; tiles are assigned so that the workgroups resident on one XCD share
// their activation and weight slabs in that XCD's L2.

#include "aq_device.h"
#include "aq_internal.h"
#include "aq_tile_xform.h"

namespace aq {
namespace {

struct BigArgs {
  const int8_t *qx;
  const int8_t *E;
  const float *Es;
  const float *sx, *bias;
  float *Y;
  int32_t *P;
  int N, K, R, C, M, MB, NB, T;
  const int8_t *useeds;  // output transform (XFORM): per tile row seed (-1 .. 6)
  OutTables ot;
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int kBM = 256, kBN = 256, kBK = 128, kNP = 8;

// Cache policy of the output stores: non-temporal (bit 1), so the FP32
// outputs, never read again here, leave the caches to the operand slabs.
constexpr int kStoreNT = 2;

// s_waitcnt: all vector-memory and LDS/scalar accesses of this wave done.
constexpr int kWaitAll = (7 << 4);

__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, const void *lds, int bytes,
                                    uint32_t voff, uint32_t soff) {
  if (bytes == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

// Tile id t (0 .. T-1) -> (bm, bn).  Workgroup b walks t = b, b + G, ...;
// hardware places workgroup b on XCD b % 8.  Within each round of G tiles,
// the tiles of XCD x are made a contiguous range of the logical order, which
// walks 8 M-blocks down one N-block column before moving right.
__device__ __forceinline__ void tile_coords(const BigArgs &a, int t, int G, int &bm, int &bn) {
  const int round0 = (t / G) * G;
  const int Gl = min(G, a.T - round0);
  const int kb = t - round0;
  const int per = Gl / 8;
  const int L = round0 + ((kb < per * 8) ? (kb % 8) * per + kb / 8 : kb);
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * a.NB;
  const int first_m = (L / in_group) * GROUP_M;
  const int gsize = min(a.MB - first_m, GROUP_M);
  bm = first_m + (L % in_group) % gsize;
  bn = (L % in_group) / gsize;
}

template <bool PARTIALS, bool XFORM>
__global__ __launch_bounds__(512, 1) void prefill_big_kernel(const BigArgs a) {
  static_assert(!(PARTIALS && XFORM), "the debug products take no output transform");
  constexpr int A_BYTES = kBM * kBK, B_BYTES = kBN * kBK;
  __shared__ __attribute__((aligned(1024))) int8_t As0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t As1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t Bs0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t Bs1[B_BYTES];
  __shared__ __attribute__((aligned(256))) float Ss0[8 * 64];   // per-wave row scales
  __shared__ __attribute__((aligned(256))) float Ss1[8 * 64];
  __shared__ __attribute__((aligned(256))) float Xs0[kBM];      // token scales of a tile
  __shared__ __attribute__((aligned(256))) float Xs1[kBM];
  __shared__ __attribute__((aligned(256))) float Xs2[kBM];
  __shared__ __attribute__((aligned(256))) float Bb0[kBN];      // bias of a tile
  __shared__ __attribute__((aligned(256))) float Bb1[kBN];
  __shared__ __attribute__((aligned(256))) float Bb2[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1;   // rows wm*128 .. +127 of the tile
  const int wn = wave >> 1;  // tile row r0 + wn (64 outputs)
  const int G = gridDim.x;
  const int C = a.C;
  const int ntiles = (a.T - (int)blockIdx.x + G - 1) / G;
  const int total = ntiles * C;

  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.qx, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rE =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.E, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rS =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.Es, 0, 0x7FFFFFFF, 0x00020000);
  // The token-scale and bias loads are issued every column, so they need a
  // valid source even when the call has none (the debug products pass no
  // token scales; most calls pass no bias): they then read qx, which holds
  // M*K >= 4M bytes, and the values are never used.
  const void *xsrc = a.sx ? (const void *)a.sx : (const void *)a.qx;
  const __amdgpu_buffer_rsrc_t rX =
      __builtin_amdgcn_make_buffer_rsrc((void *)xsrc, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.bias ? (const void *)a.bias : xsrc), 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rY =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.Y, 0, 0x7FFFFFFF, 0x00020000);
  const int bias_n = a.bias ? a.N : a.M;  // elements the bias loads may index

  // ---- per-lane constants
  // A slab: LDS chunk c = (wave*4 + i)*64 + lane is row c/8, physical chunk
  // c%8 holding logical chunk (c%8) ^ ((row >> 1) & 7).

  // B slab: wave w moves panels 4*(w&1) .. +3 of its own tile row r0 + wn.
  const uint32_t b_lane = (uint32_t)lane * 16u + (uint32_t)(wave & 1) * 4096u;
  int8_t *const b_dst0 = Bs0 + wave * 4096;
  int8_t *const b_dst1 = Bs1 + wave * 4096;
  // fragment reads: A (fm, u) at (af0 ^ 32u) + 4096 fm; B (u, fn) at
  // bf0 + 2048 u + 512 fn.
  const int af0 = (wm * 128 + l32) * kBK + ((h ^ ((l32 >> 1) & 7)) * 16);
  const int bf0 = (wn * kNP + h) * 1024 + l32 * 16;
  // epilogue: lane's part of an output offset (bytes); rows 4h, columns l32
  const uint32_t y_lane = ((uint32_t)(wm * 128 + 4 * h) * (uint32_t)a.N + (uint32_t)(wn * 64 + l32)) * 4u;

  // ---- state of the column being issued
  int iss_ti = 0, iss_j = 0;       // tile index (of this workgroup) and column
  int iss_m0 = 0, iss_r0 = 0;      // its tile's first token row and tile row
  auto set_issue_tile = [&](int ti) __attribute__((always_inline)) {
    int bm, bn;
    tile_coords(a, (int)blockIdx.x + ti * G, G, bm, bn);
    iss_m0 = bm * kBM;
    iss_r0 = bn * 4;
  };
  auto xs_buf = [&](int ti) __attribute__((always_inline)) -> float * {
    const int k = ti % 3;
    return k == 0 ? Xs0 : k == 1 ? Xs1 : Xs2;
  };
  auto bb_buf = [&](int ti) __attribute__((always_inline)) -> float * {
    const int k = ti % 3;
    return k == 0 ? Bb0 : k == 1 ? Bb1 : Bb2;
  };
  // issue the loads of column (iss_ti, iss_j) into stage st
  auto issue = [&](int st) __attribute__((always_inline)) {
    int8_t *As_ = st ? As1 : As0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (wave * 4 + i) * 64 + lane;
      const int row = c >> 3;
      const int chk = ((c & 7) ^ ((row >> 1) & 7)) * 16;
      const uint32_t voff = (uint32_t)min(iss_m0 + row, a.M - 1) * (uint32_t)a.K + (uint32_t)chk;
      dma(rq, As_ + (wave * 4 + i) * 1024, 16, voff, (uint32_t)iss_j * kBK);
    }
    const int rw = min(iss_r0 + wn, a.R - 1);
    const uint32_t bsoff = ((uint32_t)rw * (uint32_t)C + (uint32_t)iss_j) * (uint32_t)(64 * kBK);
    int8_t *b_dst = st ? b_dst1 : b_dst0;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma(rE, b_dst + i * 1024, 16, b_lane, bsoff + (uint32_t)i * 1024u);
    float *Ss_ = (st ? Ss1 : Ss0) + wave * 64;
    dma(rS, Ss_, 4, (uint32_t)lane * 4u, ((uint32_t)rw * (uint32_t)C + (uint32_t)iss_j) * 256u);
    // the tile's token scales (waves 0-3) or bias (waves 4-7), 64 per wave;
    // one unconditional load per wave, its source and target selected
    const bool xw = wave < 4;
    const int m = min(iss_m0 + wave * 64 + lane, a.M - 1);
    const int n = min(min(iss_r0 + wave - 4, a.R - 1) * 64 + lane, bias_n - 1);
    dma(xw ? rX : rB, xw ? xs_buf(iss_ti) + wave * 64 : bb_buf(iss_ti) + (wave - 4) * 64, 4,
        (uint32_t)(xw ? m : n) * 4u, 0u);
  };
  // one of the ten loads of a column (k: 0-3 activation slab, 4-7 weight
  // panels, 8 row scales, 9 token scales or bias); spread over a column's
  // first sub-tiles so the load issue does not stall the MFMA stream
  auto issue_part = [&](int st, int k) __attribute__((always_inline)) {
    if (k < 4) {
      const int c = (wave * 4 + k) * 64 + lane;
      const int row = c >> 3;
      const int chk = ((c & 7) ^ ((row >> 1) & 7)) * 16;
      const uint32_t voff = (uint32_t)min(iss_m0 + row, a.M - 1) * (uint32_t)a.K + (uint32_t)chk;
      dma(rq, (st ? As1 : As0) + (wave * 4 + k) * 1024, 16, voff, (uint32_t)iss_j * kBK);
    } else if (k < 9) {
      const int rw = min(iss_r0 + wn, a.R - 1);
      if (k < 8) {
        const uint32_t bsoff = ((uint32_t)rw * (uint32_t)C + (uint32_t)iss_j) * (uint32_t)(64 * kBK);
        dma(rE, (st ? b_dst1 : b_dst0) + (k - 4) * 1024, 16, b_lane, bsoff + (uint32_t)(k - 4) * 1024u);
      } else {
        dma(rS, (st ? Ss1 : Ss0) + wave * 64, 4, (uint32_t)lane * 4u,
            ((uint32_t)rw * (uint32_t)C + (uint32_t)iss_j) * 256u);
      }
    } else {
      const bool xw = wave < 4;
      const int m = min(iss_m0 + wave * 64 + lane, a.M - 1);
      const int n = min(min(iss_r0 + wave - 4, a.R - 1) * 64 + lane, bias_n - 1);
      dma(xw ? rX : rB, xw ? xs_buf(iss_ti) + wave * 64 : bb_buf(iss_ti) + (wave - 4) * 64, 4,
          (uint32_t)(xw ? m : n) * 4u, 0u);
    }
  };
  auto advance_issue = [&]() __attribute__((always_inline)) {
    if (iss_ti * C + iss_j + 1 < total) {
      if (++iss_j == C) {
        iss_j = 0;
        ++iss_ti;
        set_issue_tile(iss_ti);
      }
    }
  };

  float F[4][2][16];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[fm][fn][e] = 0.f;
  v16i acc[2];  // INT32 products of the current and the previous 32 x 32 sub-tile
  acc[0] = acc[1] = v16i{0};
  float scp0 = 0.f, scp1 = 0.f, scn0 = 0.f, scn1 = 0.f;

  // the finished tile ti's outputs: Y = F * sx + bias (XFORM: Y~ U on the
  // wave's tile row first, one 32-token slice at a time to bound the
  // registers of the exchange), then F = 0
  auto epilogue = [&](int ti) __attribute__((always_inline)) {
    int bm, bn;
    tile_coords(a, (int)blockIdx.x + ti * G, G, bm, bn);
    const int m0 = bm * kBM, r0 = bn * 4;
    if constexpr (XFORM) {
      const int s = a.useeds[min(r0 + wn, a.R - 1)];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) out_transform<1>(*reinterpret_cast<float(*)[1][2][16]>(&F[fm]), s, lane, a.ot);
    }
    const float *xs = xs_buf(ti) + wm * 128 + 4 * h;
    const float *bb = bb_buf(ti) + wn * 64 + l32;
    const float b0 = a.bias ? bb[0] : 0.f, b1 = a.bias ? bb[32] : 0.f;
    const bool live = r0 + wn < a.R;
    const bool full = m0 + kBM <= a.M;
    const uint32_t ybase = ((uint32_t)m0 * (uint32_t)a.N + (uint32_t)r0 * 64u) * 4u;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float4 s4 = *reinterpret_cast<const float4 *>(xs + fm * 32 + 8 * e4);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e3 = 0; e3 < 4; ++e3) {
          const int mrel = wm * 128 + fm * 32 + 8 * e4 + 4 * h + e3;  // row inside the tile
          const uint32_t soff = ybase + (uint32_t)(fm * 32 + 8 * e4 + e3) * (uint32_t)a.N * 4u;
          const float v0 = fmaf(F[fm][0][4 * e4 + e3], sv[e3], b0);
          const float v1 = fmaf(F[fm][1][4 * e4 + e3], sv[e3], b1);
          if (live && (full || m0 + mrel < a.M)) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), rY, y_lane, soff, kStoreNT);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), rY, y_lane + 128u, soff, kStoreNT);
          }
        }
      }
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e) F[fm][fn][e] = 0.f;
  };

  // rescale the INT32 products of one 32 x 32 sub-tile (register set p) of
  // fragment (fm, fn) with its rows' scale sv
// (the empty asm pins the results here: without it the compiler sinks the
// rescale below later MFMAs and keeps every sub-tile's products live)
#define AQ_RESCALE(p, fm, fn, sv)                                                     \
  do {                                                                                \
    _Pragma("unroll") for (int e = 0; e < 16; ++e)                                    \
      F[fm][fn][e] = fmaf((float)acc[p][e], (sv), F[fm][fn][e]);                      \
    _Pragma("unroll") for (int e = 0; e < 16; e += 4)                                 \
      asm volatile("" : "+v"(F[fm][fn][e]), "+v"(F[fm][fn][e + 1]),                   \
                   "+v"(F[fm][fn][e + 2]), "+v"(F[fm][fn][e + 3]));                   \
  } while (0)

  // one column of the stream; st = stage (compile-time after unrolling)
  int cur_ti = 0, cur_j = 0;
  int cur_m0 = 0, cur_r0 = 0;  // tile of the column being multiplied (debug products)
  auto column = [&](const int st) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitAll);  // this column's loads have landed ...
    __builtin_amdgcn_s_barrier();          // ... in every wave; the other stage is free
    if constexpr (PARTIALS) {
      if (cur_j == 0) {
        int bm, bn;
        tile_coords(a, (int)blockIdx.x + cur_ti * G, G, bm, bn);
        cur_m0 = bm * kBM;
        cur_r0 = bn * 4;
      }
    } else {
      if (cur_j == 0 && cur_ti > 0) epilogue(cur_ti - 1);
    }
    advance_issue();
    scp0 = scn0;
    scp1 = scn1;
    const float *Ss_ = (st ? Ss1 : Ss0) + wave * 64;
    scn0 = Ss_[l32];
    scn1 = Ss_[32 + l32];
    const int8_t *As_ = st ? As1 : As0;
    const int8_t *Bs_ = st ? Bs1 : Bs0;
    // Eight 32 x 32 sub-tiles per column, n-fragment outer: the four weight
    // fragments (k-steps) of fn stay in registers across the four m-fragments;
    // activation fragments are read one k-step ahead.  Sub-tile q's products
    // go to register set q & 1 and are rescaled during sub-tile q + 1 (the
    // column's last one during the next column's first).
    v4i fb[4], fa[3];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        fb[u] = *reinterpret_cast<const v4i *>(Bs_ + bf0 + u * 2048 + fn * 512);
      fa[0] = *reinterpret_cast<const v4i *>(As_ + af0);
      fa[1] = *reinterpret_cast<const v4i *>(As_ + (af0 ^ 32));
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
        const int q = fn * 4 + fm, p = q & 1;
        if (q < 5) {  // next column's loads, two per sub-tile
          issue_part(st ^ 1, 2 * q);
          issue_part(st ^ 1, 2 * q + 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int st_ = fm * 4 + u;  // step of this n-fragment pass, 0 .. 15
          if (st_ + 2 < 16) {          // activation fragment two steps ahead
            const int nfm = (st_ + 2) >> 2, nu = (st_ + 2) & 3;
            fa[(st_ + 2) % 3] = *reinterpret_cast<const v4i *>(As_ + (af0 ^ (32 * nu)) + nfm * 4096);
          }
          acc[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[st_ % 3], fb[u], u == 0 ? v16i{0} : acc[p], 0, 0, 0);
        }
        if constexpr (PARTIALS) {
          // 32x32 MFMA result: column (output n) = lane & 31, row (token) =
          // 8 (e / 4) + 4 (lane >> 5) + (e & 3)
          const int rw = cur_r0 + wn;
          if (rw < a.R) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int m = cur_m0 + wm * 128 + fm * 32 + 8 * (e / 4) + 4 * h + (e & 3);
              const size_t n = (size_t)rw * 64 + fn * 32 + l32;
              if (m < a.M) a.P[((size_t)m * a.N + n) * C + cur_j] = acc[p][e];
            }
          }
          continue;
        }
        // the previous sub-tile
        if (q == 0) AQ_RESCALE(1, 3, 1, scp1);
        else if (fm == 0) AQ_RESCALE(p ^ 1, 3, 0, scn0);
        else AQ_RESCALE(p ^ 1, fm - 1, fn, fn ? scn1 : scn0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        // keep each sub-tile's reads, MFMAs and rescale together: the
        // scheduler may not hoist later sub-tiles' reads (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!PARTIALS && cur_j == C - 1) {
      // the tile ends: finish its last sub-tile now, so that the next
      // column's first rescale adds nothing
      AQ_RESCALE(1, 3, 1, scn1);
      scn0 = scn1 = 0.f;
    }
    if (++cur_j == C) {
      cur_j = 0;
      ++cur_ti;
    }
  };

  // prologue: column 0 of the first tile into stage 0
  set_issue_tile(0);
  issue(0);
  for (int g = 0; g < total; g += 2) {
    column(0);
    if (g + 1 < total) column(1);
  }
  if constexpr (!PARTIALS) epilogue(ntiles - 1);
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may still be in flight at exit
#undef AQ_RESCALE
}

}  // namespace

hipError_t launch_prefill_big(const int8_t *E, const float *Es, int N, int K, const int8_t *qx,
                              const float *sx, int M, const float *bias, float *Y, int32_t *P,
                              hipStream_t stream, const int8_t *useeds, const aq_transform_tables *tables) {
  BigArgs a;
  a.qx = qx; a.E = E; a.Es = Es; a.sx = sx; a.bias = bias; a.Y = Y; a.P = P;
  a.useeds = useeds;
  a.ot = useeds && tables ? out_tables(*tables) : OutTables{};
  a.N = N; a.K = K; a.R = N / 64; a.C = K / kBK; a.M = M;
  a.MB = (M + kBM - 1) / kBM;
  a.NB = (a.R + 3) / 4;
  a.T = a.MB * a.NB;
  const int G = min(a.T, compute_units());
  if (P)
    hipLaunchKernelGGL((prefill_big_kernel<true, false>), dim3(G), dim3(512), 0, stream, a);
  else if (useeds && tables)
    hipLaunchKernelGGL((prefill_big_kernel<false, true>), dim3(G), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_big_kernel<false, false>), dim3(G), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace aq
