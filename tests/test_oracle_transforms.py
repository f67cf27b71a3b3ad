"""Pins of the oracle's tile-aligned transforms (App. B.1): the normalized
Hadamard matrix against its closed form, the FP32 butterfly order against
exact integer arithmetic, orthogonality of every seeded transform, the
identity seed, and eq. 4's exact reconstruction without quantization."""
import numpy as np
import pytest

from oracle import aq_oracle as O
from workloads import gen

TABLES = gen.transform_tables(6000)


def test_hadamard_closed_form():
    H = O.hadamard64()
    i, j = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(H, np.where(parity, -1.0, 1.0) / 8.0)
    assert np.allclose(H @ H.T, np.eye(64), atol=1e-15)


def test_fwht_order_exact_on_integers():
    rng = np.random.default_rng(1)
    for _ in range(5):
        v = rng.integers(-1000, 1000, size=64).astype(np.float32)     # sums stay exact in FP32
        want = (np.where(np.vectorize(lambda a: bin(a).count("1") & 1)(
            np.arange(64)[:, None] & np.arange(64)[None, :]), -1, 1) @ v.astype(np.int64)) / 8
        assert np.array_equal(O.fwht64_f32(v).astype(np.float64), want)


@pytest.mark.parametrize("s", range(-1, 7))
def test_seeded_transforms_orthogonal_and_fp32_close(s):
    F = O.phi(s, TABLES)
    assert np.allclose(F @ F.T, np.eye(64), atol=1e-14)
    rng = np.random.default_rng(10 + s)
    v = rng.standard_normal((5, 64)).astype(np.float32)
    got = O.phi_t_f32(v, s, TABLES).astype(np.float64)
    ref = v.astype(np.float64) @ F          # rows: v^T Phi = (Phi^T v)^T
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    if s == -1:
        assert np.array_equal(O.phi_t_f32(v, s, TABLES), v)


def test_eq4_reconstruction_without_quantization():
    rng = np.random.default_rng(2)
    M, N, K = 3, 128, 256
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    vs, us = gen.transform_seeds(rng, K // 64), gen.transform_seeds(rng, N // 64)
    Xt = O.transform_rows(X, vs, TABLES).astype(np.float64)
    Wt = O.transform_weights(W, us, vs, TABLES).astype(np.float64)
    Y = O.transform_out(Xt @ Wt.T, us, TABLES)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(Y - ref)) <= 2e-6 * np.max(np.abs(ref))


def test_tables_are_signed_permutations():
    perm, dl, dr = TABLES
    assert all(sorted(p.tolist()) == list(range(64)) for p in perm)
    assert set(np.unique(dl)) <= {-1, 1} and set(np.unique(dr)) <= {-1, 1}
