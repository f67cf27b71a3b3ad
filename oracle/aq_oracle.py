"""CPU oracle for the tile-aligned W4/W8 x A8 mixed-precision linear layer.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
definition that the HIP path is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and it shares no code, table or constant generator
with the HIP sources.

Source: "AlignQuant: Tile-Aligned Mixed-Precision Quantization for Efficient
LLM Generation" (arXiv 2610.07457), as carried by the paperz deep-dive page.
Each function names the section / equation it follows.

Notation (paper Sec. 3.1): Y = X W^T with X in R^{M x K}, W in R^{N x K}; W is
cut into equal b_N x b_K tiles, R = N / b_N tile rows, C = K / b_K tile
columns, T = R*C.  z[r, j] in {4, 8} is the precision map.

Readings taken where the pages are silent or are overridden by the task
statement:
  * weight scale: one FP32 scale per (output row n, tile column j), absmax rule
    s = max(absmax / q_max, 1e-12) computed in FP64 (App. B.2 eq. 5 and the
    1e-12 floor of eq. 6);
  * activation scale: one per token, s = max(absmax / 127, 1e-12), FP64;
  * intra-tile byte order: our own (the pages' CUTLASS order is specific to
    NVIDIA tensor cores):
      W8 tile = b_K/16 panels; panel p holds, for every tile row i in order,
        the 16 codes k = 16p .. 16p+15 (one byte each);
      W4 tile = b_K/32 panels; panel p holds, for every tile row i in order,
        16 bytes; byte b packs q0 = code at k = 32p + b and q1 = code at
        k = 32p + 16 + b as (q0 mod 16) + 16 (q1 mod 16)   (App. E.1 eq. 17).

The pages' own activation quantizer (App. B.3: 64-feature x b_M-row
groups, the endpoint scale of eq. 6) is here as quant_act_grouped with its
eq. 19 counterpart; the per-token form above is the default path.

Parity status: every function here is pinned by tests/test_oracle_*.py
(hand-worked fixtures under tests/golden/, closed forms, brute force and
invariants).  The pages print no per-layer input/output example, so no pin
of the linear outputs uses numbers printed there; those outputs are pinned by
the hand-worked 2 x 2-tile fixture, brute-force sums and the textbook
special cases (uniform maps, a single tile column).
"""

from __future__ import annotations

import math

import numpy as np

# App. B.2: q_min,b = -2^(b-1), q_max,b = 2^(b-1) - 1.
def qrange(b: int) -> tuple[int, int]:
    """Integer code range of a b-bit symmetric quantizer (App. B.2)."""
    if b not in (4, 8):
        raise ValueError("precision must be 4 or 8")
    return -(2 ** (b - 1)), 2 ** (b - 1) - 1


SCALE_FLOOR = 1e-12  # App. B.2 eq. 6: the scale is never below 1e-12.


# --------------------------------------------------------------------------
# Geometry and labels (Sec. 3.1; App. E.1)
# --------------------------------------------------------------------------

def tile_grid(N: int, K: int, bN: int, bK: int) -> tuple[int, int]:
    """Number of tile rows R and tile columns C (Sec. 3.1 tile partition)."""
    if N % bN or K % bK:
        raise ValueError("N and K must be multiples of the tile size")
    if bK % 32:
        raise ValueError("b_K must be a multiple of 32 for the packed layout")
    return N // bN, K // bK


def labels_from_map(zmap: np.ndarray) -> np.ndarray:
    """1-bit precision labels, 1 for W4 and 0 for W8, in row-major tile order,
    eight labels per byte with the first label in the least significant bit
    (App. E.1)."""
    R, C = zmap.shape
    T = R * C
    out = np.zeros((T + 7) // 8, dtype=np.uint8)
    for r in range(R):
        for j in range(C):
            t = r * C + j
            if zmap[r, j] == 4:
                out[t // 8] |= np.uint8(1 << (t % 8))
            elif zmap[r, j] != 8:
                raise ValueError("precision map entries must be 4 or 8")
    return out


def map_from_labels(labels: np.ndarray, R: int, C: int) -> np.ndarray:
    """Inverse of labels_from_map (App. E.1)."""
    z = np.empty((R, C), dtype=np.int64)
    for r in range(R):
        for j in range(C):
            t = r * C + j
            z[r, j] = 4 if (int(labels[t // 8]) >> (t % 8)) & 1 else 8
    return z


def row_offsets(zmap: np.ndarray, b: int) -> np.ndarray:
    """INT32[R+1]: number of b-bit tiles in tile rows before r (App. E.1
    eq. 16 'stored row offset'; App. E.2 length R+1)."""
    R, _ = zmap.shape
    off = np.zeros(R + 1, dtype=np.int32)
    for r in range(R):
        off[r + 1] = off[r] + int(np.sum(zmap[r] == b))
    return off


def tile_index(zmap: np.ndarray, r: int, j: int) -> int:
    """Physical index of tile (r, j) inside the buffer of its own precision
    (App. E.1 eq. 16): same-precision tiles in earlier rows plus those before
    column j in row r."""
    b = int(zmap[r, j])
    before_rows = sum(int(zmap[rr, jj] == b) for rr in range(r)
                      for jj in range(zmap.shape[1]))
    in_row = sum(int(zmap[r, jj] == b) for jj in range(j))
    return before_rows + in_row


def int8_tile_count(frac8: float, T: int) -> int:
    """Tile count from a fraction, nearest integer with ties to even
    (App. D.4 rounding of k = round(rho |T|))."""
    return int(round(frac8 * T))  # Python's round() is half-to-even


# --------------------------------------------------------------------------
# Quantizers (App. B.2 eq. 5-6; App. B.3)
# --------------------------------------------------------------------------

def quantize(A: np.ndarray, s: float, b: int) -> np.ndarray:
    """Q_b(A; s) = clip(round_even(A / s), q_min, q_max), zero point 0
    (App. B.2 eq. 5).  Division and rounding in FP64."""
    lo, hi = qrange(b)
    A64 = np.asarray(A, dtype=np.float64)
    s64 = np.asarray(s, dtype=np.float64)
    return np.clip(np.rint(A64 / s64), lo, hi).astype(np.int64)


def absmax_scale(A: np.ndarray, b: int) -> float:
    """max(max|A| / q_max,b, 1e-12) in FP64 (absmax form of the scale with the
    floor of App. B.2 eq. 6)."""
    _, hi = qrange(b)
    a = float(np.max(np.abs(np.asarray(A, dtype=np.float64)))) if np.size(A) else 0.0
    return max(a / hi, SCALE_FLOOR)


def quant_weights(W: np.ndarray, zmap: np.ndarray, bN: int, bK: int):
    """Per-tile-row weight quantization.

    For tile (r, j) with precision b = z[r, j] and each row n of that tile the
    FP64 scale s = max(absmax(W[n, tile cols]) / q_max,b, 1e-12) gives codes
    Q_b(W[n, tile cols]; s); the stored scale is FP32(s) (App. B.2: integer
    construction in FP64, s_b,t = FP32(s*)).

    Returns codes int64 [N, K] and sW float32 [N, C].
    """
    N, K = W.shape
    R, C = tile_grid(N, K, bN, bK)
    codes = np.zeros((N, K), dtype=np.int64)
    sW = np.zeros((N, C), dtype=np.float32)
    for r in range(R):
        for j in range(C):
            b = int(zmap[r, j])
            _, hi = qrange(b)
            rows = slice(r * bN, (r + 1) * bN)
            cols = slice(j * bK, (j + 1) * bK)
            seg = np.asarray(W[rows, cols], dtype=np.float64)      # [bN, bK]
            s = np.maximum(np.max(np.abs(seg), axis=1) / hi, SCALE_FLOOR)  # [bN]
            codes[rows, cols] = quantize(seg, s[:, None], b)
            sW[rows, j] = s.astype(np.float32)
    return codes, sW


def mse_scale(A: np.ndarray, b: int) -> float:
    """s*_b(A) of App. B.2 eq. 7: over the grid s_i = max((1/4 + i/128)
    s_0,b(A), 1e-12), i = 0 .. 128, the s_i minimizing ||A - s_i Q_b(A; s_i)||^2,
    the first such i on equal errors (grid order).  FP64; the squared error
    is summed element by element in index order, each product and sum
    rounded on its own (no fused multiply-add), so that the choice is fixed
    to the last bit."""
    A64 = np.asarray(A, dtype=np.float64).ravel()
    s0 = endpoint_scale(A64, b)
    best_s, best_e = None, None
    for i in range(129):
        s = max((0.25 + i / 128) * s0, SCALE_FLOOR)
        d = A64 - s * quantize(A64, s, b).astype(np.float64)
        e = float(np.cumsum(d * d)[-1]) if d.size else 0.0
        if best_e is None or e < best_e:
            best_s, best_e = s, e
    return best_s


def quant_weights_mse(W: np.ndarray, zmap: np.ndarray, bN: int, bK: int):
    """Per-tile-row weight quantization with the fitted scale of App. B.2
    eq. 7 (grid around eq. 6's endpoint scale) in place of the absmax scale:
    for tile (r, j) of precision b and each row n of it, s = s*_b(W[n, tile
    cols]), codes Q_b(W[n, tile cols]; s), stored scale FP32(s).  Returns
    codes int64 [N, K] and sW float32 [N, C]."""
    N, K = W.shape
    R, C = tile_grid(N, K, bN, bK)
    codes = np.zeros((N, K), dtype=np.int64)
    sW = np.zeros((N, C), dtype=np.float32)
    for r in range(R):
        for j in range(C):
            b = int(zmap[r, j])
            for n in range(r * bN, (r + 1) * bN):
                seg = np.asarray(W[n, j * bK:(j + 1) * bK], dtype=np.float64)
                s = mse_scale(seg, b)
                codes[n, j * bK:(j + 1) * bK] = quantize(seg, s, b)
                sW[n, j] = np.float32(s)
    return codes, sW


def quant_act(X: np.ndarray):
    """Per-token INT8 activation quantization: for row m,
    s = max(max_k |X[m,k]| / 127, 1e-12) in FP64, qx = Q_8(X[m]; s), and the
    stored scale is FP32(s) (App. B.3 computes in FP64 and stores INT8 codes
    with FP32 scales; eq. 5 rounding)."""
    X = np.asarray(X)
    M, K = X.shape
    qx = np.zeros((M, K), dtype=np.int64)
    sx = np.zeros(M, dtype=np.float32)
    for m in range(M):
        row = X[m].astype(np.float64)
        s = absmax_scale(row, 8)
        qx[m] = quantize(row, s, 8)
        sx[m] = np.float32(s)
    return qx, sx


# --------------------------------------------------------------------------
# Tile-aligned orthogonal transforms (App. B.1, eq. 4)
# --------------------------------------------------------------------------
#
# Phi_-1 = I, Phi_0 = H_64 (the normalized 64-point Hadamard matrix, entries
# +-1/8), Phi_s = D_L,s P_s H_64 D_R,s for s = 1 .. 6, with P_s a permutation
# and D_L,s, D_R,s diagonal sign matrices.  The pages do not say how P_s and
# the signs follow from s; here they are inputs, `tables` = (perm, dl, dr)
# with perm[s-1] a permutation of 0..63 ((P v)_i = v[perm[i]]) and dl[s-1],
# dr[s-1] vectors of +-1.  V = diag(Phi_{v_c}) over 64-feature blocks and
# U = diag(Phi_{u_r}^T) over 64-row output tile rows.

TB = 64  # transform block (the pages' 64 x 64 configuration)


def hadamard64() -> np.ndarray:
    """H_64 in Sylvester (natural) order, normalized: entries +-1/8, FP64."""
    H = np.array([[1.0]])
    while H.shape[0] < TB:
        H = np.block([[H, H], [H, -H]])
    return H / 8.0


def phi(s: int, tables) -> np.ndarray:
    """The seeded 64 x 64 transform Phi_s of App. B.1, FP64."""
    if s == -1:
        return np.eye(TB)
    if s == 0:
        return hadamard64()
    perm, dl, dr = tables
    P = np.eye(TB)[np.asarray(perm[s - 1])]
    return np.diag(np.asarray(dl[s - 1], np.float64)) @ P @ hadamard64() @ np.diag(np.asarray(dr[s - 1], np.float64))


def fwht64_f32(v: np.ndarray) -> np.ndarray:
    """H_64 v in FP32, by the in-place butterflies in order h = 1, 2, 4, ...,
    32 ((a_i, a_i+h) -> (a_i + a_i+h, a_i - a_i+h) for i with bit h clear),
    then the exact scaling by 1/8: the evaluation order both sides use so
    that transformed values are identical to the last bit.  Acts on the
    last axis."""
    a = np.array(v, dtype=np.float32, copy=True)
    h = 1
    while h < TB:
        idx = np.arange(TB)
        lo = idx[(idx & h) == 0]
        x, y = a[..., lo].copy(), a[..., lo + h].copy()
        a[..., lo] = x + y
        a[..., lo + h] = x - y
        h *= 2
    return a * np.float32(0.125)


def phi_t_f32(v: np.ndarray, s: int, tables) -> np.ndarray:
    """Phi_s^T v in FP32 along the last axis: D_R H (P^T (D_L v)); the sign
    flips, the permutation and the 1/8 are exact, only the butterflies
    round."""
    v = np.asarray(v, dtype=np.float32)
    if s == -1:
        return v.copy()
    if s == 0:
        return fwht64_f32(v)
    perm, dl, dr = tables
    u = v * np.asarray(dl[s - 1], np.float32)
    w = np.empty_like(u)
    w[..., np.asarray(perm[s - 1])] = u            # P^T: w[perm[i]] = u[i]
    return fwht64_f32(w) * np.asarray(dr[s - 1], np.float32)


def transform_rows(X: np.ndarray, seeds, tables) -> np.ndarray:
    """X~ = X V (App. B.1): every 64-feature block c of every row becomes
    Phi_{v_c}^T x (x as a column), FP32."""
    X = np.asarray(X, dtype=np.float32)
    out = np.empty_like(X)
    for c, sd in enumerate(seeds):
        out[..., TB * c:TB * (c + 1)] = phi_t_f32(X[..., TB * c:TB * (c + 1)], int(sd), tables)
    return out


def transform_weights(W: np.ndarray, useeds, vseeds, tables) -> np.ndarray:
    """W~ = U W V (App. B.1), FP32: first each row's 64-feature blocks
    (W V), then each 64-row tile row's columns by U_r = Phi_{u_r}^T."""
    Wv = transform_rows(W, vseeds, tables)
    out = np.empty_like(Wv)
    for r, sd in enumerate(useeds):
        blk = Wv[TB * r:TB * (r + 1), :]                       # [64, K]
        out[TB * r:TB * (r + 1), :] = phi_t_f32(blk.T, int(sd), tables).T
    return out


def transform_out(Yt: np.ndarray, useeds, tables) -> np.ndarray:
    """Y = Y~ U (App. B.1 eq. 4), FP64: every 64-feature output block r of
    every row becomes Phi_{u_r} y~ (U_r = Phi_{u_r}^T acting on row vectors)."""
    Yt = np.asarray(Yt, dtype=np.float64)
    out = np.empty_like(Yt)
    for r, sd in enumerate(useeds):
        out[:, TB * r:TB * (r + 1)] = Yt[:, TB * r:TB * (r + 1)] @ phi(int(sd), tables).T
    return out


# --------------------------------------------------------------------------
# The pages' activation quantizer (App. B.3 with App. B.2 eq. 5-6)
# --------------------------------------------------------------------------

ACT_GROUP_K = 64   # App. B.3: one activation scale per 64 features ...


def act_group_rows(M: int) -> int:
    """... and b_M rows: b_M = 1 when M = 1, otherwise 16 (App. B.3)."""
    return 1 if M == 1 else 16


def endpoint_scale(A: np.ndarray, b: int) -> float:
    """s_0,b(A) = max(max(0, max A) / q_max,b, max(0, -min A) / |q_min,b|,
    1e-12) in FP64 (App. B.2 eq. 6)."""
    lo, hi = qrange(b)
    A64 = np.asarray(A, dtype=np.float64)
    top = max(0.0, float(np.max(A64))) if A64.size else 0.0
    bot = max(0.0, -float(np.min(A64))) if A64.size else 0.0
    return max(top / hi, bot / abs(lo), SCALE_FLOOR)


def quant_act_grouped(X: np.ndarray):
    """The pages' activation quantization (App. B.3): rows are zero-padded to
    M' = ceil(M / b_M) b_M; every group A of b_M rows x 64 features gets the
    FP64 scale s = s_0,8(A) of eq. 6 and codes Q_8(A; s) (eq. 5); the stored
    scale is FP32(s).  Padding rows are zero, so they change no group's
    maximum or minimum beyond the zeros eq. 6 already includes; the codes of
    the padding rows are dropped (the output is sliced back to M rows).

    Returns qx int64 [M, K] and sxg float32 [ceil(M / b_M), K / 64], group
    (g, c) covering rows g b_M .. g b_M + b_M - 1 and features 64c .. 64c+63.
    """
    X = np.asarray(X)
    M, K = X.shape
    if K % ACT_GROUP_K:
        raise ValueError("K must be a multiple of 64")
    bM = act_group_rows(M)
    G = -(-M // bM)
    Xp = np.zeros((G * bM, K), dtype=np.float64)
    Xp[:M] = X
    qx = np.zeros((G * bM, K), dtype=np.int64)
    sxg = np.zeros((G, K // ACT_GROUP_K), dtype=np.float32)
    for g in range(G):
        for c in range(K // ACT_GROUP_K):
            rows = slice(g * bM, (g + 1) * bM)
            cols = slice(c * ACT_GROUP_K, (c + 1) * ACT_GROUP_K)
            A = Xp[rows, cols]
            s = endpoint_scale(A, 8)
            qx[rows, cols] = quantize(A, s, 8)
            sxg[g, c] = np.float32(s)
    return qx[:M], sxg


def group_partials(qx: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """P[m, n, c] = sum over the 64 features k of activation group c of
    qx[m, k] * codes[n, k]: eq. 19's integer product per 64-wide column
    group (a b_K = 128 tile holds two), int64 [M, N, K / 64].  Each product
    is a float64 matrix product of integers below 2^53, hence exact."""
    return tile_partials(qx, codes, ACT_GROUP_K)


def linear_from_group_partials(P: np.ndarray, sxg: np.ndarray, sW: np.ndarray, bK: int,
                               bias: np.ndarray | None = None) -> np.ndarray:
    """y[m, n] = sum_c s^X_{g(m), c} s^W_{n, j(c)} P[m, n, c] (+ bias[n]) in
    FP64, c in increasing order, g(m) = m // b_M and j(c) = 64 c // b_K the
    tile column holding group c (App. E.3 eq. 19 with the App. B.3 groups)."""
    M, N, CG = P.shape
    bM = act_group_rows(M)
    sx64 = np.asarray(sxg, dtype=np.float64)[np.arange(M) // bM]     # [M, CG]
    sW64 = np.asarray(sW, dtype=np.float64)
    y = np.zeros((M, N), dtype=np.float64)
    for c in range(CG):
        j = (c * ACT_GROUP_K) // bK
        y += (sx64[:, c][:, None] * sW64[None, :, j]) * P[:, :, c].astype(np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y


def abs_contrib_grouped(P: np.ndarray, sxg: np.ndarray, sW: np.ndarray, bK: int) -> np.ndarray:
    """sum_c |s^X_{g(m), c} s^W_{n, j(c)} P[m, n, c]|, the componentwise
    error scale of an FP32 evaluation of the grouped eq. 19."""
    M, N, CG = P.shape
    bM = act_group_rows(M)
    sx64 = np.asarray(sxg, dtype=np.float64)[np.arange(M) // bM]
    sW64 = np.asarray(sW, dtype=np.float64)
    a = np.zeros((M, N), dtype=np.float64)
    for c in range(CG):
        j = (c * ACT_GROUP_K) // bK
        a += np.abs((sx64[:, c][:, None] * sW64[None, :, j]) * P[:, :, c].astype(np.float64))
    return a


# --------------------------------------------------------------------------
# Packing (Sec. 3.2; App. E.1 eq. 16-17; App. E.2)
# --------------------------------------------------------------------------

def pack_tile_w8(tile_codes: np.ndarray) -> np.ndarray:
    """Bytes of one W8 tile: b_K/16 panels, each holding 16 codes per tile row
    (rows in order), one two's-complement byte per code."""
    bN, bK = tile_codes.shape
    out = np.zeros((bK // 16, bN, 16), dtype=np.uint8)
    for p in range(bK // 16):
        out[p] = (tile_codes[:, 16 * p:16 * p + 16] % 256).astype(np.uint8)
    return out.reshape(-1)


def nibble_byte(q0, q1):
    """byte(q0, q1) = (q0 mod 16) + 16 (q1 mod 16)  (App. E.1 eq. 17)."""
    return (np.asarray(q0) % 16) + 16 * (np.asarray(q1) % 16)


def nibble_value(v):
    """A nibble v expands to v if v < 8 and to v - 16 otherwise (App. E.1)."""
    v = np.asarray(v)
    return np.where(v < 8, v, v - 16)


def pack_tile_w4(tile_codes: np.ndarray) -> np.ndarray:
    """Bytes of one W4 tile: b_K/32 panels, each holding 16 bytes per tile row
    (rows in order); byte b of a row's 16 packs the codes at k = 32p + b and
    k = 32p + 16 + b by eq. 17."""
    bN, bK = tile_codes.shape
    lo, hi = qrange(4)
    if tile_codes.min(initial=0) < lo or tile_codes.max(initial=0) > hi:
        raise ValueError("INT4 code out of range")
    out = np.zeros((bK // 32, bN, 16), dtype=np.uint8)
    for p in range(bK // 32):
        q0 = tile_codes[:, 32 * p:32 * p + 16]
        q1 = tile_codes[:, 32 * p + 16:32 * p + 32]
        out[p] = nibble_byte(q0, q1).astype(np.uint8)
    return out.reshape(-1)


def unpack_tile_w8(buf: np.ndarray, bN: int, bK: int) -> np.ndarray:
    panels = buf.reshape(bK // 16, bN, 16).astype(np.int64)
    codes = np.zeros((bN, bK), dtype=np.int64)
    for p in range(bK // 16):
        codes[:, 16 * p:16 * p + 16] = np.where(panels[p] < 128, panels[p], panels[p] - 256)
    return codes


def unpack_tile_w4(buf: np.ndarray, bN: int, bK: int) -> np.ndarray:
    panels = buf.reshape(bK // 32, bN, 16).astype(np.int64)
    codes = np.zeros((bN, bK), dtype=np.int64)
    for p in range(bK // 32):
        codes[:, 32 * p:32 * p + 16] = nibble_value(panels[p] % 16)
        codes[:, 32 * p + 16:32 * p + 32] = nibble_value(panels[p] // 16)
    return codes


def pack(codes: np.ndarray, sW: np.ndarray, zmap: np.ndarray, bN: int, bK: int) -> dict:
    """Split W4/W8 packed representation (Sec. 3.2; App. E.1-E.2).

    Selected W4 and W8 tiles go to two contiguous buffers in row order; tile
    (r, j) sits at index_b(r, j) of eq. 16 in the buffer of its precision; its
    b_N per-row FP32 scales sit at the same index in s4 / s8.  Returns a dict
    with labels, row_off4, row_off8, w4 (uint8 [T4*bN*bK/2]),
    w8 (uint8 [T8*bN*bK]), s4 (float32 [T4*bN]), s8 (float32 [T8*bN]).
    """
    N, K = codes.shape
    R, C = tile_grid(N, K, bN, bK)
    T4 = int(np.sum(zmap == 4))
    T8 = int(np.sum(zmap == 8))
    w4 = np.zeros(T4 * bN * bK // 2, dtype=np.uint8)
    w8 = np.zeros(T8 * bN * bK, dtype=np.uint8)
    s4 = np.zeros(T4 * bN, dtype=np.float32)
    s8 = np.zeros(T8 * bN, dtype=np.float32)
    off4 = row_offsets(zmap, 4)
    off8 = row_offsets(zmap, 8)
    for r in range(R):
        seen4 = 0
        seen8 = 0
        for j in range(C):
            tile = codes[r * bN:(r + 1) * bN, j * bK:(j + 1) * bK]
            scales = sW[r * bN:(r + 1) * bN, j]
            if zmap[r, j] == 4:
                idx = int(off4[r]) + seen4
                seen4 += 1
                nb = bN * bK // 2
                w4[idx * nb:(idx + 1) * nb] = pack_tile_w4(tile)
                s4[idx * bN:(idx + 1) * bN] = scales
            else:
                idx = int(off8[r]) + seen8
                seen8 += 1
                nb = bN * bK
                w8[idx * nb:(idx + 1) * nb] = pack_tile_w8(tile)
                s8[idx * bN:(idx + 1) * bN] = scales
    return dict(labels=labels_from_map(zmap), row_off4=off4, row_off8=off8,
                w4=w4, w8=w8, s4=s4, s8=s8, N=N, K=K, bN=bN, bK=bK, T4=T4, T8=T8)


def unpack(packed: dict):
    """Inverse of pack: returns codes int64 [N, K], sW float32 [N, C] and the
    precision map, locating every tile from its logical coordinate through
    its label, its row offset and eq. 16 (App. E.1)."""
    N, K, bN, bK = packed["N"], packed["K"], packed["bN"], packed["bK"]
    R, C = tile_grid(N, K, bN, bK)
    zmap = map_from_labels(packed["labels"], R, C)
    codes = np.zeros((N, K), dtype=np.int64)
    sW = np.zeros((N, C), dtype=np.float32)
    for r in range(R):
        for j in range(C):
            b = int(zmap[r, j])
            off = packed["row_off4"] if b == 4 else packed["row_off8"]
            pos = sum(int(zmap[r, jj] == b) for jj in range(j))
            idx = int(off[r]) + pos
            if b == 4:
                nb = bN * bK // 2
                tile = unpack_tile_w4(packed["w4"][idx * nb:(idx + 1) * nb], bN, bK)
                sc = packed["s4"][idx * bN:(idx + 1) * bN]
            else:
                nb = bN * bK
                tile = unpack_tile_w8(packed["w8"][idx * nb:(idx + 1) * nb], bN, bK)
                sc = packed["s8"][idx * bN:(idx + 1) * bN]
            codes[r * bN:(r + 1) * bN, j * bK:(j + 1) * bK] = tile
            sW[r * bN:(r + 1) * bN, j] = sc
    return codes, sW, zmap


def pack_weights(W: np.ndarray, zmap: np.ndarray, bN: int, bK: int) -> dict:
    """Quantize then pack (App. B.2 followed by App. E.1)."""
    codes, sW = quant_weights(W, zmap, bN, bK)
    return pack(codes, sW, zmap, bN, bK)


# --------------------------------------------------------------------------
# Tile products and output reconstruction (Sec. 3.3; App. E.3 eq. 19)
# --------------------------------------------------------------------------

def tile_partials(qx: np.ndarray, codes: np.ndarray, bK: int) -> np.ndarray:
    """P[m, n, j] = sum over k in tile column j of qx[m, k] * codes[n, k]: the
    parenthesized integer tile product of eq. 19, int64 [M, N, C].

    Each product is formed with a float64 matrix product: every term and
    partial sum is an integer below 2^53, so the result is exact."""
    M, K = qx.shape
    N, K2 = codes.shape
    if K != K2 or K % bK:
        raise ValueError("shape mismatch")
    C = K // bK
    P = np.zeros((M, N, C), dtype=np.int64)
    for j in range(C):
        a = qx[:, j * bK:(j + 1) * bK].astype(np.float64)
        w = codes[:, j * bK:(j + 1) * bK].astype(np.float64)
        P[:, :, j] = np.rint(a @ w.T).astype(np.int64)
    if P.size and (P.max() > 2**31 - 1 or P.min() < -2**31):
        raise OverflowError("tile partial exceeds INT32")
    return P


def linear_from_partials(P: np.ndarray, sx: np.ndarray, sW: np.ndarray,
                         bias: np.ndarray | None = None) -> np.ndarray:
    """y[m, n] = sum_j s^X_m s^W_{n,j} P[m, n, j] (+ bias[n]) in FP64,
    j in increasing order (App. E.3 eq. 19; interface adds bias when present)."""
    M, N, C = P.shape
    y = np.zeros((M, N), dtype=np.float64)
    sx64 = np.asarray(sx, dtype=np.float64)
    sW64 = np.asarray(sW, dtype=np.float64)
    for j in range(C):
        y += (sx64[:, None] * sW64[None, :, j]) * P[:, :, j].astype(np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y


def abs_contrib(P: np.ndarray, sx: np.ndarray, sW: np.ndarray) -> np.ndarray:
    """sum_j |s^X_m s^W_{n,j} P[m, n, j]|: the scale of the rounding error an
    FP32 evaluation of eq. 19 can make; used by the componentwise gate."""
    M, N, C = P.shape
    a = np.zeros((M, N), dtype=np.float64)
    sx64 = np.asarray(sx, dtype=np.float64)
    sW64 = np.asarray(sW, dtype=np.float64)
    for j in range(C):
        a += np.abs((sx64[:, None] * sW64[None, :, j]) * P[:, :, j].astype(np.float64))
    return a


def linear(X: np.ndarray, W: np.ndarray, zmap: np.ndarray, bN: int, bK: int,
           bias: np.ndarray | None = None) -> np.ndarray:
    """The whole path: quantize weights and activations, integer tile
    products, FP64 rescale and sum (Sec. 3.3)."""
    codes, sW = quant_weights(W, zmap, bN, bK)
    qx, sx = quant_act(X)
    return linear_from_partials(tile_partials(qx, codes, bK), sx, sW, bias)


# --------------------------------------------------------------------------
# Storage accounting (App. E.2 eq. 18)
# --------------------------------------------------------------------------

def packed_bytes_paper(T4: int, T8: int, R: int, C: int, bN: int, bK: int) -> int:
    """S_packed = B/2 T4 + B T8 + 4 (T4 + T8) + ceil(RC/8) + 8 (R+1), with
    one FP32 scale per tile (App. E.2 eq. 18)."""
    B = bN * bK
    return B * T4 // 2 + B * T8 + 4 * (T4 + T8) + math.ceil(R * C / 8) + 8 * (R + 1)


def packed_bytes_rowscale(T4: int, T8: int, R: int, C: int, bN: int, bK: int) -> int:
    """Eq. 18 with one FP32 scale per tile row instead of per tile: the scale
    term becomes 4 b_N (T4 + T8)."""
    B = bN * bK
    return B * T4 // 2 + B * T8 + 4 * bN * (T4 + T8) + math.ceil(R * C / 8) + 8 * (R + 1)


def bits_per_weight(S_packed: int, T4: int, T8: int, bN: int, bK: int) -> float:
    """Complete packed bits per weight 8 S / (B (T4 + T8)) (App. E.2)."""
    return 8.0 * S_packed / (bN * bK * (T4 + T8))
