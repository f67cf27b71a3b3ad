"""The seeded generators are deterministic and produce the stated shapes and
INT8 fractions."""
import numpy as np

from workloads import gen


def test_small_is_seeded_and_shaped():
    a, b = gen.small(), gen.small()
    assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["X"], b["X"])
    assert a["W"].shape == (256, 512) and a["X"].shape == (4, 512)
    assert int(np.sum(a["zmap"] == 8)) == 8 and int(np.sum(a["zmap"] == 4)) == 8


def test_llama3b_fractions():
    for proj, N, K in gen.LLAMA3B:
        d = gen.llama3b_decode(proj, 1)
        R, C = N // 64, K // 128
        assert d["zmap"].shape == (R, C)
        assert int(np.sum(d["zmap"] == 8)) == int(round(0.25 * R * C))


def test_bands_are_contiguous_rows():
    rng = np.random.default_rng(0)
    z = gen.map_bands(rng, 96, 20, 0.30)
    assert int(np.sum(z == 8)) == int(round(0.3 * 96 * 20))
    full = [r for r in range(96) if np.all(z[r] == 8)]
    part = [r for r in range(96) if 0 < np.sum(z[r] == 8) < 20]
    assert len(full) == (576 // 20) and len(part) == 1
    runs = 1 + sum(1 for a, b in zip(full, full[1:]) if b != a + 1)
    assert runs <= 4


def test_model_weighted_budget():
    maps = gen.qwen14b_maps()
    T = sum(m.size for layer in maps for m in layer)
    T8 = sum(int(np.sum(m == 8)) for layer in maps for m in layer)
    assert T8 == int(round(0.3 * T))
