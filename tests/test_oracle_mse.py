"""Pins of the oracle's fitted weight scale (App. B.2 eq. 7, around eq. 6's
endpoint scale): exact rational arithmetic over the same grid, closed forms
for representable and zero segments, and the endpoint scale as an upper
bound of the error."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import aq_oracle as O


def exact_argmin(A, b):
    """Eq. 7 in exact rational arithmetic: (error, i, s) of the first grid
    point with the least error."""
    lo, hi = O.qrange(b)
    A = [Fraction(float(x)) for x in A]
    floor = Fraction(1e-12)
    s0 = max(max(Fraction(0), max(A)) / hi, max(Fraction(0), -min(A)) / abs(lo), floor)
    best = None
    for i in range(129):
        s = max((Fraction(1, 4) + Fraction(i, 128)) * s0, floor)
        err = Fraction(0)
        for a in A:
            q = a / s
            f = q.numerator // q.denominator
            rem = q - f
            if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2):
                f += 1
            err += (a - s * min(max(f, lo), hi)) ** 2
        if best is None or err < best[0]:
            best = (err, i, s)
    return best


@pytest.mark.parametrize("b", [4, 8])
@pytest.mark.parametrize("seed", range(6))
def test_fp64_choice_equals_exact_argmin(b, seed):
    rng = np.random.default_rng(100 * b + seed)
    A = rng.standard_normal(16) * rng.choice([0.01, 1.0, 5.0]) * (1 + 9 * (rng.random(16) < 0.1))
    _, i, _ = exact_argmin(A, b)
    # the same grid point: FP64 evaluates it from the rounded endpoint scale
    assert O.mse_scale(A, b) == max((0.25 + i / 128) * O.endpoint_scale(A, b), 1e-12)


def test_hand_case():
    # [127, 1.5] at 8 bits: s0 = 1; larger scales trade a little error on 127
    # for less on 1.5; the exact minimum is at i = 126, s = 79/64
    assert exact_argmin([127.0, 1.5], 8)[1:] == (126, Fraction(79, 64))
    assert O.mse_scale(np.array([127.0, 1.5]), 8) == 79 / 64


@pytest.mark.parametrize("b", [4, 8])
def test_representable_segment_keeps_endpoint_scale(b):
    lo, hi = O.qrange(b)
    s = 0.0123
    Q = np.array([lo, hi, 0, 1, -1, 3] * 5 + [lo, hi], dtype=np.float64)
    A = s * Q
    assert O.endpoint_scale(A, b) == max(A.max() / hi, -A.min() / abs(lo))
    assert O.mse_scale(A, b) == O.endpoint_scale(A, b)   # i = 96, zero error


def test_zero_segment_and_bound():
    assert O.mse_scale(np.zeros(32), 8) == 1e-12
    rng = np.random.default_rng(3)
    for b in (4, 8):
        A = rng.standard_normal(128)
        s = O.mse_scale(A, b)
        e = lambda t: float(np.sum((A - t * O.quantize(A, t, b)) ** 2))
        assert e(s) <= e(O.endpoint_scale(A, b)) + 1e-15
        grid = [(0.25 + i / 128) * O.endpoint_scale(A, b) for i in range(129)]
        assert any(s == g for g in grid)


def test_quant_weights_mse_shapes_and_ranges():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((8, 256)) * 0.02
    z = np.array([[4, 8], [8, 4]])
    codes, sW = O.quant_weights_mse(W, z, 4, 128)
    assert codes.shape == W.shape and sW.shape == (8, 2)
    for r in range(2):
        for j in range(2):
            lo, hi = O.qrange(int(z[r, j]))
            blk = codes[4 * r:4 * r + 4, 128 * j:128 * j + 128]
            assert blk.min() >= lo and blk.max() <= hi
            for n in range(4 * r, 4 * r + 4):
                assert sW[n, j] == np.float32(O.mse_scale(W[n, 128 * j:128 * j + 128], int(z[r, j])))
