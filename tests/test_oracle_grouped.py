"""Pins of the oracle's grouped activation quantizer (App. B.3: 64-feature x
b_M-row groups with the endpoint scale of App. B.2 eq. 6) and of its eq. 19
counterpart, against closed forms, a hand-worked case, the padding rule and
a brute-force dequantize-then-matmul."""
import json
import os

import numpy as np
import pytest

from oracle import aq_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_endpoint_rule_closed_forms():
    # both endpoints binding: 127 and -128 are reached exactly
    t = 0.37
    A = np.zeros((1, 64)); A[0, 3] = 127 * t; A[0, 9] = -128 * t
    q, s = O.quant_act_grouped(A)
    assert float(s[0, 0]) == np.float32(t)
    assert q[0, 3] == 127 and q[0, 9] == -128
    # positive side decides: s = max A / 127
    A = np.zeros((1, 64)); A[0, 0] = 254.0; A[0, 1] = -10.0
    q, s = O.quant_act_grouped(A)
    assert float(s[0, 0]) == 2.0 and q[0, 0] == 127 and q[0, 1] == -5
    # negative side decides: s = -min A / 128
    A = np.zeros((1, 64)); A[0, 0] = 10.0; A[0, 1] = -256.0
    q, s = O.quant_act_grouped(A)
    assert float(s[0, 0]) == 2.0 and q[0, 0] == 5 and q[0, 1] == -128
    # all-zero group: the 1e-12 floor, zero codes
    q, s = O.quant_act_grouped(np.zeros((1, 128)))
    assert np.all(s == np.float32(1e-12)) and not q.any()
    # one-sided groups: max(0, .) keeps the other side out
    A = np.full((1, 64), -3.0)
    q, s = O.quant_act_grouped(A)
    assert float(s[0, 0]) == np.float32(3.0 / 128) and np.all(q == -128)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "grouped_act_hand.json")))
    X = np.zeros((1, 128)); W = np.zeros((1, 128))
    for v, k in g["x"].items():
        X[0, k] = float(v)
    for v, k in g["w"].items():
        W[0, k] = float(v)
    qx, sxg = O.quant_act_grouped(X)
    for k, v in g["qx_nonzero"].items():
        assert qx[0, int(k)] == v
    assert int(np.count_nonzero(qx)) == len(g["qx_nonzero"])
    assert np.array_equal(sxg[0], np.array(g["sxg"], dtype=np.float32))
    codes, sW = O.quant_weights(W, np.array([[8]]), 1, 128)
    assert codes[0, 0] == 64 and codes[0, 64] == 127
    P = O.group_partials(qx, codes)
    assert P[0, 0].tolist() == g["P"]
    y = O.linear_from_group_partials(P, sxg, sW, 128)
    # FP32-stored scales: within a few FP32 ulps of the exact -380/127
    assert abs(y[0, 0] - g["y_num"] / g["y_den"]) <= 1e-6


@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 40])
def test_group_rows_and_padding(M):
    rng = np.random.default_rng(M)
    K = 192
    X = rng.standard_normal((M, K)) * rng.choice([0.1, 1.0, 30.0], size=K)[None, :]
    q, s = O.quant_act_grouped(X)
    bM = 1 if M == 1 else 16
    assert s.shape == (-(-M // bM), K // 64)
    for g in range(s.shape[0]):
        rows = X[g * bM:min(M, (g + 1) * bM)]
        for c in range(K // 64):
            A = rows[:, 64 * c:64 * c + 64]
            want = max(max(0.0, A.max()) / 127, max(0.0, -A.min()) / 128, 1e-12)
            assert s[g, c] == np.float32(want)
    if M > 1:
        # explicit zero padding to a multiple of 16 rows changes nothing
        Xp = np.zeros((-(-M // 16) * 16, K)); Xp[:M] = X
        qp, sp = O.quant_act_grouped(Xp)
        assert np.array_equal(sp, s) and np.array_equal(qp[:M], q)


def test_grouped_linear_equals_dequantized_matmul():
    """Brute force: eq. 19 over 64-wide groups equals dequantize-then-matmul
    (both in FP64, rounding order aside), for both tile widths, mixed maps
    and 1 or several rows."""
    rng = np.random.default_rng(5)
    for (N, K, bN, bK, M) in [(8, 256, 4, 128, 1), (8, 256, 4, 128, 5), (6, 192, 3, 64, 18), (4, 128, 2, 128, 33)]:
        W = rng.standard_normal((N, K)) * 0.05
        z = rng.choice([4, 8], size=(N // bN, K // bK))
        X = rng.standard_normal((M, K)) * rng.choice([1.0, 20.0], size=K)[None, :]
        codes, sW = O.quant_weights(W, z, bN, bK)
        qx, sxg = O.quant_act_grouped(X)
        y = O.linear_from_group_partials(O.group_partials(qx, codes), sxg, sW, bK)
        bM = O.act_group_rows(M)
        Xd = qx * np.repeat(np.asarray(sxg, np.float64)[np.arange(M) // bM], 64, axis=1)
        Wd = codes * np.repeat(np.asarray(sW, np.float64), bK, axis=1)
        ref = Xd @ Wd.T
        assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        # the error bound that gates the GPU outputs is never smaller than |y|
        c = O.abs_contrib_grouped(O.group_partials(qx, codes), sxg, sW, bK)
        assert np.all(c + 1e-300 >= np.abs(y) * (1 - 1e-12))


def test_grouped_codes_stay_in_range_and_round_half_even():
    s = 0.5
    A = np.zeros((1, 64)); A[0, :4] = [0.25, 0.75, -0.25, 63.5]   # /s -> 0.5, 1.5, -0.5, 127
    q, sx = O.quant_act_grouped(A)
    assert float(sx[0, 0]) == s
    assert q[0, :4].tolist() == [0, 2, 0, 127]
    rng = np.random.default_rng(0)
    q, _ = O.quant_act_grouped(rng.standard_normal((33, 256)) * 50)
    assert q.min() >= -128 and q.max() <= 127
