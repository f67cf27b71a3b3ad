"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every check here is independent of the oracle's own arithmetic: hand-derived
fixtures under tests/golden/ (each cites its passage), closed forms, brute
force on tiny inputs and invariants.  test_planted_mistakes_are_caught plants
plausible mistakes in the oracle (on the CPU) and asserts that a pin fails.
"""
import json
import os

import numpy as np
import pytest

from oracle import aq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _dense(shape, nonzero, dtype=np.float64):
    a = np.zeros(shape, dtype=dtype)
    for e in nonzero:
        a[tuple(e[:-1])] = e[-1]
    return a


# ---------------------------------------------------------------- fixtures

def check_hand_2x2():
    g = _gold("hand_2x2.json")
    N, K, bN, bK = g["N"], g["K"], g["bN"], g["bK"]
    z = np.array(g["zmap"])
    W = _dense((N, K), g["W_nonzero"])
    X = _dense((1, K), g["X_nonzero"])
    pk = O.pack_weights(W, z, bN, bK)
    assert list(pk["labels"]) == g["labels"]
    assert list(pk["row_off4"]) == g["row_off4"]
    assert list(pk["row_off8"]) == g["row_off8"]
    assert np.array_equal(pk["w4"], _dense((g["w4_len"],), g["w4_nonzero_bytes"]).astype(np.uint8))
    assert np.array_equal(pk["w8"], _dense((g["w8_len"],), g["w8_nonzero_bytes"]).astype(np.uint8))
    assert list(pk["s4"]) == g["s4"] and list(pk["s8"]) == g["s8"]
    qx, sx = O.quant_act(X)
    assert np.array_equal(qx, _dense((1, K), g["qx_nonzero"]).astype(np.int64))
    assert list(sx) == g["sx"]
    codes, sW, _ = O.unpack(pk)
    P = O.tile_partials(qx, codes, bK)
    assert P.tolist() == g["P"]
    y = O.linear_from_partials(P, sx, sW)
    assert y.tolist() == g["y"]
    assert O.linear(X, W, z, bN, bK).tolist() == g["y"]


def test_hand_2x2():
    check_hand_2x2()


def check_panel_order():
    g = _gold("panel_order.json")
    N, K, bN, bK = g["N"], g["K"], g["bN"], g["bK"]
    z = np.array(g["zmap"])
    codes = np.zeros((N, K), dtype=np.int64)
    k = np.arange(32)
    codes[0, :32] = k
    codes[1, :32] = -1 - k
    codes[0, 32:48] = np.arange(16) - 8
    codes[0, 48:64] = 7 - np.arange(16)
    codes[1, 32:64] = -1
    codes[1, 32] = 5
    codes[1, 63] = -8
    sW = np.ones((N, 2), dtype=np.float32)
    pk = O.pack(codes, sW, z, bN, bK)
    assert list(pk["labels"]) == g["labels"]
    assert list(pk["row_off4"]) == g["row_off4"] and list(pk["row_off8"]) == g["row_off8"]
    assert pk["w8"].tobytes().hex() == g["w8_hex"].replace(" ", "")
    assert pk["w4"].tobytes().hex() == g["w4_hex"].replace(" ", "")
    back, _, zb = O.unpack(pk)
    assert np.array_equal(back, codes) and np.array_equal(zb, z)


def test_panel_order():
    check_panel_order()


def check_eq16():
    g = _gold("eq16_index.json")
    ex = g["worked_example"]
    z = np.array(ex["zmap"])
    for j, want in enumerate(ex["index"][0]):
        assert O.tile_index(z, 0, j) == want
    c = g["case_3x3"]
    z = np.array(c["zmap"])
    assert list(O.row_offsets(z, 4)) == c["row_off4"]
    assert list(O.row_offsets(z, 8)) == c["row_off8"]
    assert list(O.labels_from_map(z)) == c["labels"]
    for r in range(3):
        for j in range(3):
            assert O.tile_index(z, r, j) == c["index"][r][j]
    # The packed buffers hold each tile at that index: pack distinct constant
    # tiles and read them back by the fixture's index.
    bN, bK = 1, 32
    codes = np.zeros((3, 96), dtype=np.int64)
    for r in range(3):
        for j in range(3):
            codes[r, j * 32:(j + 1) * 32] = 3 * r + j - 4   # in [-4, 4]
    pk = O.pack(codes, np.ones((3, 3), np.float32), z, bN, bK)
    for r in range(3):
        for j in range(3):
            idx = c["index"][r][j]
            if z[r, j] == 4:
                byte = int(pk["w4"][idx * 16])
                v = 3 * r + j - 4
                assert byte == ((v & 15) | ((v & 15) << 4))
            else:
                assert int(np.int8(pk["w8"][idx * 32].view(np.int8))) == 3 * r + j - 4


def test_eq16_index():
    check_eq16()


# ---------------------------------------------------------------- eq. 17

def check_eq17():
    for q0 in range(-8, 8):
        for q1 in range(-8, 8):
            byte = int(O.nibble_byte(q0, q1))
            # two's-complement nibbles written with bit operations
            assert byte == ((q0 & 0xF) | ((q1 & 0xF) << 4))
            assert 0 <= byte < 256
            assert int(O.nibble_value(byte & 0xF)) == q0
            assert int(O.nibble_value(byte >> 4)) == q1


def test_eq17_all_pairs():
    check_eq17()


def test_label_bit_order_lsb_first():
    R, C = 3, 5
    for t in range(R * C):
        z = np.full((R, C), 8)
        z[t // C, t % C] = 4
        lab = O.labels_from_map(z)
        bits = [(int(lab[i // 8]) >> (i % 8)) & 1 for i in range(len(lab) * 8)]
        assert bits.index(1) == t and sum(bits) == 1
        assert np.array_equal(O.map_from_labels(lab, R, C), z)


# ---------------------------------------------------------------- eq. 18

def test_table16_packed_bpw():
    g = _gold("table16_bpw.json")
    bN, bK = g["tile"]
    # Llama-3.2-3B-shaped projections (fused qkv, o, fused gate_up, down);
    # to two decimals the result does not depend on the layer count.
    projs = [(5120, 3072), (3072, 3072), (16384, 3072), (3072, 8192)]
    for layers in (1, 28):
        geo = [(N // bN, K // bK) for N, K in projs] * layers
        T = sum(R * C for R, C in geo)
        for rho, want in zip(g["w4_fraction"], g["packed_bpw"]):
            T4 = O.int8_tile_count(rho, T)   # same rounding rule for any fraction
            T8 = T - T4
            # eq. 18 per projection, splitting T4 proportionally is not needed:
            # only the totals enter the integer and scale terms.
            S = 0
            left4 = T4
            for R, C in geo:
                t4 = min(left4, R * C)
                left4 -= t4
                S += O.packed_bytes_paper(t4, R * C - t4, R, C, bN, bK)
            bpw = O.bits_per_weight(S, T4, T8, bN, bK)
            assert round(bpw, 2) == want
            # integer-weight cost 8 - 4 rho_real plus ~33/(bN bK) metadata (F.2)
            assert abs(bpw - (8 - 4 * T4 / T) - 33 / (bN * bK)) < 1e-3


def test_eq18_closed_form_components():
    # one W4 and one W8 64x128 tile in one row: bytes add up term by term
    S = O.packed_bytes_paper(1, 1, 1, 2, 64, 128)
    assert S == 4096 + 8192 + 8 + 1 + 16
    S2 = O.packed_bytes_rowscale(1, 1, 1, 2, 64, 128)
    assert S2 - S == 4 * 64 * 2 - 8


def test_tile_count_half_even():
    assert O.int8_tile_count(0.5, 5) == 2      # 2.5 -> 2
    assert O.int8_tile_count(0.5, 7) == 4      # 3.5 -> 4
    assert O.int8_tile_count(0.25, 10) == 2    # 2.5 -> 2
    assert O.int8_tile_count(0.0, 10) == 0 and O.int8_tile_count(1.0, 10) == 10


# ---------------------------------------------------------------- quantizers

def check_quantize_ties():
    assert O.quantize(np.array([-2.5, 0.5, 63.5, 1.5, -0.5, 2.5]), 1.0, 8).tolist() == [-2, 0, 64, 2, 0, 2]
    assert O.quantize(np.array([7.5, -8.5, 100.0, -100.0, 6.5]), 1.0, 4).tolist() == [7, -8, 7, -8, 6]
    assert O.quantize(np.array([200.0, -200.0, 127.5, -128.5]), 1.0, 8).tolist() == [127, -128, 127, -128]
    assert O.qrange(4) == (-8, 7) and O.qrange(8) == (-128, 127)


def test_quantize_ties_and_clip():
    check_quantize_ties()


def check_weight_scale_properties(seed=0):
    rng = np.random.default_rng(seed)
    bN, bK = 4, 64
    W = rng.standard_normal((8, 128)) * 0.02
    W[1, :64] = 0.0                              # an all-zero tile row
    z = np.array([[4, 8], [8, 4]])
    codes, sW = O.quant_weights(W, z, bN, bK)
    for r in range(2):
        for j in range(2):
            qmax = 7 if z[r, j] == 4 else 127
            for i in range(bN):
                n = r * bN + i
                seg = W[n, j * bK:(j + 1) * bK]
                q = codes[n, j * bK:(j + 1) * bK]
                if not np.any(seg):
                    assert sW[n, j] == np.float32(1e-12) and not np.any(q)
                    continue
                # absmax element maps to +-q_max with its sign
                a = np.argmax(np.abs(seg))
                assert q[a] == np.sign(seg[a]) * qmax
                assert np.abs(q).max() == qmax
                # every code is the nearest integer of w / s (scale recovered
                # from the stored FP32 value to within its rounding)
                s = float(sW[n, j])
                assert abs(np.abs(seg).max() / s - qmax) < 1e-5 * qmax
                assert np.all(np.abs(seg / s - q) <= 0.5 + 1e-4)


def test_weight_scale_properties():
    check_weight_scale_properties()


def test_quant_act_properties():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 96)).astype(np.float32)
    X[2] = 0.0
    X[3, 7] = -40.0
    qx, sx = O.quant_act(X)
    assert sx[2] == np.float32(1e-12) and not np.any(qx[2])
    for m in (0, 1, 3, 4):
        a = np.argmax(np.abs(X[m]))
        assert qx[m, a] == np.sign(X[m, a]) * 127
        assert np.all(np.abs(X[m] / float(sx[m]) - qx[m]) <= 0.5 + 1e-4)
    assert qx.min() >= -128 and qx.max() <= 127


def test_int4_codes_in_range():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((64, 256)) * 0.02
    W[5, 3] = 1.0                                  # outlier
    z = np.full((1, 2), 4)
    codes, _ = O.quant_weights(W, z, 64, 128)
    assert codes.min() >= -8 and codes.max() <= 7
    assert codes.min() >= -7                       # absmax scale never reaches -8


# ---------------------------------------------------------------- packing

def test_roundtrip_random_codes_full_range():
    rng = np.random.default_rng(3)
    for (N, K, bN, bK) in [(64, 128, 64, 128), (128, 256, 64, 64), (6, 96, 3, 32), (1, 32, 1, 32)]:
        R, C = N // bN, K // bK
        z = rng.choice([4, 8], size=(R, C))
        codes = np.zeros((N, K), dtype=np.int64)
        for r in range(R):
            for j in range(C):
                lo, hi = (-8, 7) if z[r, j] == 4 else (-128, 127)
                codes[r * bN:(r + 1) * bN, j * bK:(j + 1) * bK] = rng.integers(lo, hi + 1, size=(bN, bK))
        sW = rng.random((N, C)).astype(np.float32)
        pk = O.pack(codes, sW, z, bN, bK)
        assert pk["w4"].size == pk["T4"] * bN * bK // 2 and pk["w8"].size == pk["T8"] * bN * bK
        c2, s2, z2 = O.unpack(pk)
        assert np.array_equal(c2, codes) and np.array_equal(s2, sW) and np.array_equal(z2, z)


def test_int4_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_tile_w4(np.full((1, 32), 8))


# ---------------------------------------------------------------- products

def _brute_partials(qx, codes, bK):
    M, K = qx.shape
    N = codes.shape[0]
    P = np.zeros((M, N, K // bK), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            for k in range(K):
                P[m, n, k // bK] += int(qx[m, k]) * int(codes[n, k])
    return P


def check_partials_brute(seed=4):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-128, 128, size=(3, 64))
    codes = rng.integers(-128, 128, size=(5, 64))
    assert np.array_equal(O.tile_partials(qx, codes, 32), _brute_partials(qx, codes, 32))
    # extreme magnitudes stay exact
    qx = np.full((1, 128), -128)
    codes = np.full((2, 128), -128)
    assert O.tile_partials(qx, codes, 128)[0, 0, 0] == 128 * 128 * 128


def test_partials_brute_force():
    check_partials_brute()


def check_dequant_matmul(seed=5, bias=True):
    rng = np.random.default_rng(seed)
    N, K, bN, bK, M = 12, 96, 4, 32, 3
    W = rng.standard_normal((N, K)) * 0.02
    X = rng.standard_normal((M, K))
    X[:, 5] *= 20
    z = rng.choice([4, 8], size=(N // bN, K // bK))
    b = rng.standard_normal(N) if bias else None
    y = O.linear(X, W, z, bN, bK, b)
    codes, sW = O.quant_weights(W, z, bN, bK)
    qx, sx = O.quant_act(X)
    # textbook dequantize-then-matmul in FP64
    Wd = codes.astype(np.float64) * np.repeat(sW.astype(np.float64), bK, axis=1)
    Xd = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    yb = Xd @ Wd.T + (b if bias else 0.0)
    assert np.max(np.abs(y - yb)) <= 1e-12 * np.max(np.abs(yb))
    # and the quantized layer approximates the float layer
    yf = X @ W.T + (b if bias else 0.0)
    assert np.max(np.abs(y - yf)) < 0.2 * np.max(np.abs(yf - (b if bias else 0.0)))


def test_dequant_matmul_brute_force():
    check_dequant_matmul()
    check_dequant_matmul(seed=6, bias=False)


def _textbook_w8a8_per_channel(X, W):
    """Per-channel W8A8: one absmax/127 scale per output row and per token."""
    sw = np.maximum(np.abs(W).max(axis=1) / 127.0, 1e-12)
    qw = np.clip(np.rint(W / sw[:, None]), -128, 127)
    sx = np.maximum(np.abs(X).max(axis=1) / 127.0, 1e-12)
    qx = np.clip(np.rint(X / sx[:, None]), -128, 127)
    acc = qx @ qw.T                       # exact in FP64 at these sizes
    return acc * sx.astype(np.float32).astype(np.float64)[:, None] * \
        sw.astype(np.float32).astype(np.float64)[None, :]


def test_all_int8_single_tile_column_is_per_channel_w8a8():
    rng = np.random.default_rng(7)
    N, K, M = 8, 64, 4
    W = rng.standard_normal((N, K)) * 0.02
    X = rng.standard_normal((M, K))
    z = np.full((2, 1), 8)                # b_N = 4, b_K = K -> C = 1
    y = O.linear(X, W, z, 4, K)
    yt = _textbook_w8a8_per_channel(X, W)
    assert np.max(np.abs(y - yt)) <= 1e-12 * np.max(np.abs(yt))


def test_uniform_maps_are_grouped_quantization():
    """All-INT8 (all-INT4) maps equal W8A8 (W4A8) with one weight scale per
    (row, b_K group), quantized here without tiles or packing."""
    rng = np.random.default_rng(8)
    N, K, bK, M = 8, 128, 32, 2
    W = rng.standard_normal((N, K)) * 0.02
    X = rng.standard_normal((M, K))
    sx = np.maximum(np.abs(X).max(axis=1) / 127.0, 1e-12)
    qx = np.clip(np.rint(X / sx[:, None]), -128, 127)
    for bits, qmax in ((8, 127), (4, 7)):
        Wg = W.reshape(N, K // bK, bK)
        sw = np.maximum(np.abs(Wg).max(axis=2) / qmax, 1e-12)
        qw = np.clip(np.rint(Wg / sw[:, :, None]), -qmax - 1, qmax)
        yt = np.einsum("mgk,ngk,ng->mn", qx.reshape(M, K // bK, bK), qw,
                       sw.astype(np.float32).astype(np.float64)) * \
            sx.astype(np.float32).astype(np.float64)[:, None]
        z = np.full((N // 4, K // bK), bits)
        y = O.linear(X, W, z, 4, bK)
        assert np.max(np.abs(y - yt)) <= 1e-12 * np.max(np.abs(yt))


def test_partials_linear_in_codes():
    rng = np.random.default_rng(9)
    a = rng.integers(-60, 60, size=(2, 64))
    b = rng.integers(-60, 60, size=(2, 64))
    w = rng.integers(-128, 128, size=(3, 64))
    assert np.array_equal(O.tile_partials(a + b, w, 32),
                          O.tile_partials(a, w, 32) + O.tile_partials(b, w, 32))


def test_storage_order_does_not_change_output():
    """Two maps with the same per-tile precisions produce the same Y whatever
    the packed order: Y from unpack(pack(.)) equals Y from the codes."""
    rng = np.random.default_rng(10)
    N, K, bN, bK = 8, 128, 4, 32
    W = rng.standard_normal((N, K)) * 0.02
    X = rng.standard_normal((2, K))
    z = rng.choice([4, 8], size=(2, 4))
    codes, sW = O.quant_weights(W, z, bN, bK)
    c2, s2, _ = O.unpack(O.pack(codes, sW, z, bN, bK))
    qx, sx = O.quant_act(X)
    y1 = O.linear_from_partials(O.tile_partials(qx, codes, bK), sx, sW)
    y2 = O.linear_from_partials(O.tile_partials(qx, c2, bK), sx, s2)
    assert np.array_equal(y1, y2)


def check_abs_contrib_hand():
    """The componentwise error scale of eq. 19 (sum of the terms' magnitudes),
    per token and with the App. B.3 groups, on hand-worked values."""
    g = _gold("abs_contrib_hand.json")
    t = g["per_token"]
    got = O.abs_contrib(np.array(t["P"]), np.array(t["sx"], np.float32), np.array(t["sW"], np.float32))
    assert got.tolist() == t["expected"]
    h = _gold("hand_2x2.json")
    P = np.array(h["P"])
    sW = np.array([[1.0, 1.0], [1.0, 0.5]], np.float32)   # rows' scales of the 2x2 fixture
    assert O.abs_contrib(P, np.array(h["sx"], np.float32), sW).tolist() == g["hand_2x2"]["expected"]
    gr = g["grouped"]
    sxg, sWg = np.array(gr["sxg"], np.float32), np.array(gr["sW"], np.float32)
    assert O.abs_contrib_grouped(np.array(gr["P_one_token"]), sxg, sWg, 64).tolist() == gr["expected_one_token_bk64"]
    assert O.abs_contrib_grouped(np.array(gr["P_four_groups"]), np.array(gr["sxg_four_groups"], np.float32),
                                 sWg, 128).tolist() == gr["expected_four_groups_bk128"]
    assert O.abs_contrib_grouped(np.array(gr["P_two_tokens"]), sxg, sWg, 64).tolist() == \
        gr["expected_two_tokens_bk64"]


def test_abs_contrib_hand():
    check_abs_contrib_hand()


def check_mse_hand():
    """Eq. 7 fitted scales and the codes they give, on hand-worked segments at
    8 and 4 bits whose fitted codes differ from the absmax codes."""
    g = _gold("mse_scale_hand.json")
    W = _dense((g["N"], g["K"]), g["W_nonzero"])
    codes, sW = O.quant_weights_mse(W, np.array(g["zmap"]), g["bN"], g["bK"])
    assert np.array_equal(codes, _dense((g["N"], g["K"]), g["codes_nonzero"]).astype(np.int64))
    assert sW.tolist() == g["sW"]
    # the absmax route gives other codes on the same segments
    ca, _ = O.quant_weights(W, np.array(g["zmap"]), g["bN"], g["bK"])
    assert np.array_equal(ca, _dense((g["N"], g["K"]), g["absmax_codes_nonzero"]).astype(np.int64))


def test_mse_hand():
    check_mse_hand()


def test_empty_token_batch():
    qx, sx = O.quant_act(np.zeros((0, 64), np.float32))
    assert qx.shape == (0, 64) and sx.shape == (0,)
    P = O.tile_partials(qx, np.zeros((4, 64), np.int64), 32)
    assert P.shape == (0, 4, 2)
    assert O.linear_from_partials(P, sx, np.ones((4, 2), np.float32)).shape == (0, 4)


# ---------------------------------------------------------------- mutations

def _expect_failure(fn):
    try:
        fn()
    except (AssertionError, ValueError):
        return True
    return False


MUTATIONS = {
    "no_nibble_sign_extension": ("nibble_value", lambda v: np.asarray(v)),
    "swapped_nibbles": ("nibble_byte", lambda q0, q1: (np.asarray(q1) % 16) + 16 * (np.asarray(q0) % 16)),
    "labels_msb_first": ("labels_from_map", lambda z: np.array(
        [int("".join("1" if z.reshape(-1)[t] == 4 else "0"
                     for t in range(i * 8, min(i * 8 + 8, z.size))).ljust(8, "0"), 2)
         for i in range((z.size + 7) // 8)], dtype=np.uint8)),
    "round_half_away": ("quantize", lambda A, s, b: np.clip(
        np.sign(np.asarray(A, np.float64) / s) * np.floor(np.abs(np.asarray(A, np.float64) / s) + 0.5),
        *O.qrange(b)).astype(np.int64)),
    "w4_qmax_8": ("qrange", lambda b: (-(2 ** (b - 1)), 2 ** (b - 1))),
    "partials_transposed_tile": ("tile_partials", lambda qx, codes, bK: np.stack(
        [qx[:, j * bK:(j + 1) * bK] @ codes[:, j * bK:(j + 1) * bK].T
         for j in range(qx.shape[1] // bK)][::-1], axis=2)),
    "epilogue_drops_act_scale": ("linear_from_partials", lambda P, sx, sW, bias=None: sum(
        sW[None, :, j].astype(np.float64) * P[:, :, j] for j in range(P.shape[2])) +
        (0 if bias is None else bias)),
    "epilogue_drops_bias": ("linear_from_partials", lambda P, sx, sW, bias=None: sum(
        (np.asarray(sx, np.float64)[:, None] * np.asarray(sW, np.float64)[None, :, j]) * P[:, :, j]
        for j in range(P.shape[2]))),
    "abs_contrib_drops_abs": ("abs_contrib", lambda P, sx, sW: sum(
        (np.asarray(sx, np.float64)[:, None] * np.asarray(sW, np.float64)[None, :, j]) * P[:, :, j]
        for j in range(P.shape[2]))),
    "abs_contrib_drops_act_scale": ("abs_contrib", lambda P, sx, sW: sum(
        np.abs(np.asarray(sW, np.float64)[None, :, j] * P[:, :, j]) for j in range(P.shape[2]))),
    "abs_contrib_grouped_tile_of_group": ("abs_contrib_grouped", lambda P, sxg, sW, bK: sum(
        np.abs(np.asarray(sxg, np.float64)[np.arange(P.shape[0]) // O.act_group_rows(P.shape[0])][:, c][:, None]
               * np.asarray(sW, np.float64)[None, :, min(c, sW.shape[1] - 1)] * P[:, :, c])
        for c in range(P.shape[2]))),
    "mse_codes_with_absmax_scale": ("quant_weights_mse", lambda W, z, bN, bK: (
        O.quant_weights(W, z, bN, bK)[0],
        np.array([[np.float32(O.mse_scale(W[n, j * bK:(j + 1) * bK], int(z[n // bN, j])))
                   for j in range(W.shape[1] // bK)] for n in range(W.shape[0])], np.float32))),
}

PIN_CHECKS = [check_quantize_ties, check_hand_2x2, check_panel_order, check_eq16, check_eq17,
              check_abs_contrib_hand, check_mse_hand,
              check_weight_scale_properties, check_partials_brute,
              lambda: check_dequant_matmul(5, True)]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    caught = [_expect_failure(chk) for chk in PIN_CHECKS]
    assert any(caught), f"planted mistake {name} passed every pin"
