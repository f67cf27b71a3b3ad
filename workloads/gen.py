"""Seeded synthetic inputs for the tile-aligned W4/W8 x A8 linear layer.

This module only draws random numbers: weights, activations and precision
maps of the workload shapes.  It holds none of the method's arithmetic (no
quantization, packing or products) and serves both the CPU oracle and the HIP
path, which never import each other.

Workloads (all synthetic, random init; the pages' own evaluation uses trained
checkpoints that are not available here):
  small    : one 256x512 linear, 64x128 tiles (16 tiles), 8 INT8 + 8 INT4,
             W ~ N(0, 0.02), X: M=4 tokens ~ N(0,1) with 2 channels x20.
  llama3b  : Llama-3.2-3B-shaped decode linears (fused qkv 5120x3072,
             o 3072x3072, fused gate_up 16384x3072, down 3072x8192), 25% INT8
             tiles uniformly placed, M in {1, 4, 16}, X ~ N(0,1) with 1% of
             channels x30.
  qwen4b   : Qwen3-4B-shaped prefill linears (qkv 6144x2560, o 2560x4096,
             gate_up 19456x2560, down 2560x9728), M = 2048, 30% INT8 tiles in
             4 contiguous bands of tile rows, X ~ N(0,1) with 5% of channels
             drawn from Student-t (nu = 3).
  dense8b  : 8B-class model (hidden 4096, 32 q / 8 kv heads x 128, FFN 14336,
             36 layers): per-layer INT8 fraction ~ U(0.15, 0.45).
  qwen14b  : Qwen3-14B-shaped (hidden 5120, 40 q / 8 kv heads x 128,
             FFN 17408, 40 layers): model-wide 30% INT8, sampling weighted 3x
             toward o/down tiles (Efraimidis-Spirakis keys).
"""

from __future__ import annotations

import numpy as np

TILE = (64, 128)  # default b_N x b_K

LLAMA3B = [("qkv", 5120, 3072), ("o", 3072, 3072), ("gate_up", 16384, 3072), ("down", 3072, 8192)]
QWEN4B = [("qkv", 6144, 2560), ("o", 2560, 4096), ("gate_up", 19456, 2560), ("down", 2560, 9728)]
DENSE8B = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
QWEN14B = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)]
DENSE8B_LAYERS = 36
QWEN14B_LAYERS = 40
PROJ_ID = {"qkv": 0, "o": 1, "gate_up": 2, "down": 3}


def seed_for(config: int, layer: int = 0, proj: str | int = 0) -> int:
    """Seed base 1000*config + 16*layer + projection id."""
    pid = PROJ_ID[proj] if isinstance(proj, str) else int(proj)
    return 1000 * config + 16 * layer + pid


def act_seed(config: int, layer: int = 0, proj: str | int = 0, salt: int = 0) -> int:
    """Seed of one activation input (a batch or prefill chunk `salt`):
    disjoint from every weight seed, which stay below 10^6."""
    return 1_000_000 * (1 + salt) + seed_for(config, layer, proj)


def count_from_fraction(frac: float, T: int) -> int:
    """Number of INT8 tiles for a fraction: nearest integer, ties to even."""
    return int(round(frac * T))


# ---------------------------------------------------------------- maps

def map_uniform(rng: np.random.Generator, R: int, C: int, frac8: float) -> np.ndarray:
    """int8 [R, C] of 4/8: round(frac8*T) INT8 tiles placed uniformly without
    replacement, the rest INT4."""
    T = R * C
    z = np.full(T, 4, dtype=np.int8)
    z[rng.permutation(T)[:count_from_fraction(frac8, T)]] = 8
    return z.reshape(R, C)


def map_bands(rng: np.random.Generator, R: int, C: int, frac8: float, nbands: int = 4) -> np.ndarray:
    """INT8 tiles clustered in contiguous output-channel bands: floor(T8/C)
    full tile rows split into `nbands` near-equal runs at seeded,
    non-overlapping starts, plus the first (T8 mod C) tiles of one more row."""
    T = R * C
    T8 = count_from_fraction(frac8, T)
    full, rem = divmod(T8, C)
    z = np.full((R, C), 4, dtype=np.int8)
    nb = max(1, min(nbands, full)) if full else 0
    lengths = [full // nb + (1 if i < full % nb else 0) for i in range(nb)] if nb else []
    free = R - full - (1 if rem else 0)          # rows left as gaps
    # split the free rows into nb+1 random gaps (seeded)
    cuts = np.sort(rng.integers(0, free + 1, size=nb)) if nb else np.array([], dtype=np.int64)
    gaps = np.diff(np.concatenate([[0], cuts])) if nb else np.array([], dtype=np.int64)
    row = 0
    for g, ln in zip(gaps, lengths):
        row += int(g)
        z[row:row + ln, :] = 8
        row += ln
    if rem:
        # the partial row goes to the first all-INT4 row after the bands
        cand = [r for r in range(R) if np.all(z[r] == 4)]
        z[cand[int(rng.integers(0, len(cand)))], :rem] = 8
    return z


def map_model_weighted(rng: np.random.Generator, geoms: list[tuple[int, int, float]],
                       frac8: float) -> list[np.ndarray]:
    """Model-wide budget: round(frac8 * T_total) INT8 tiles drawn by weighted
    sampling without replacement (Efraimidis-Spirakis keys u^(1/w), largest
    keys win).  geoms = [(R, C, weight)] per projection; returns the maps."""
    sizes = [R * C for R, C, _ in geoms]
    T = sum(sizes)
    w = np.concatenate([np.full(s, wt, dtype=np.float64) for s, (_, _, wt) in zip(sizes, geoms)])
    keys = rng.random(T) ** (1.0 / w)
    chosen = np.argsort(-keys, kind="stable")[:count_from_fraction(frac8, T)]
    flat = np.full(T, 4, dtype=np.int8)
    flat[chosen] = 8
    out, o = [], 0
    for (R, C, _), s in zip(geoms, sizes):
        out.append(flat[o:o + s].reshape(R, C))
        o += s
    return out


# ---------------------------------------------------------------- tensors

def weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    return (rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def acts_outliers(rng: np.random.Generator, M: int, K: int, n_out: int, mult: float) -> np.ndarray:
    """N(0,1) activations with n_out seeded outlier channels scaled by mult."""
    X = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, size=n_out, replace=False)
    X[:, ch] *= np.float32(mult)
    return X


def acts_heavy_tail(rng: np.random.Generator, M: int, K: int, frac: float = 0.05, nu: float = 3.0) -> np.ndarray:
    """N(0,1) activations where a seeded 5% of channels are Student-t(nu)."""
    X = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, size=max(1, int(round(frac * K))), replace=False)
    X[:, ch] = rng.standard_t(nu, size=(M, ch.size)).astype(np.float32)
    return X


# ---------------------------------------------------------------- workloads

def transform_tables(seed: int = 6000):
    """The six signed permutations of the seeded block transforms: perm
    uint8 [6, 64] (each row a permutation of 0..63), dl and dr int8 [6, 64]
    of +-1.  Random draws only; what they mean is defined by the consumers."""
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(64) for _ in range(6)]).astype(np.uint8)
    dl = rng.choice(np.array([-1, 1], dtype=np.int8), size=(6, 64))
    dr = rng.choice(np.array([-1, 1], dtype=np.int8), size=(6, 64))
    return perm, dl, dr


def transform_seeds(rng: np.random.Generator, n: int) -> np.ndarray:
    """n block seeds drawn uniformly from -1 .. 6 (int8)."""
    return rng.integers(-1, 7, size=n).astype(np.int8)


def small(seed: int = 1000) -> dict:
    """One 256x512 linear, 16 tiles of 64x128, 8 INT8 / 8 INT4, M = 4."""
    rng = np.random.default_rng(seed)
    bN, bK = TILE
    N, K, M = 256, 512, 4
    W = weights(rng, N, K)
    z = np.full(16, 4, dtype=np.int8)
    z[rng.permutation(16)[:8]] = 8
    X = acts_outliers(rng, M, K, 2, 20.0)
    return dict(W=W, zmap=z.reshape(N // bN, K // bK), X=X, bN=bN, bK=bK, name="small")


def llama3b_decode(proj: str, M: int, seed: int | None = None, tile=TILE) -> dict:
    """One Llama-3.2-3B-shaped decode linear with 25% INT8 tiles."""
    name, N, K = next(p for p in LLAMA3B if p[0] == proj)
    rng = np.random.default_rng(seed_for(2, 0, proj) if seed is None else seed)
    bN, bK = tile
    W = weights(rng, N, K)
    z = map_uniform(rng, N // bN, K // bK, 0.25)
    X = acts_outliers(rng, M, K, int(round(0.01 * K)), 30.0)
    return dict(W=W, zmap=z, X=X, bN=bN, bK=bK, name=f"llama3b.{name}.M{M}")


def qwen4b_prefill(proj: str, M: int = 2048, seed: int | None = None, tile=TILE) -> dict:
    """One Qwen3-4B-shaped prefill linear with 30% INT8 tiles in bands."""
    name, N, K = next(p for p in QWEN4B if p[0] == proj)
    rng = np.random.default_rng(seed_for(3, 0, proj) if seed is None else seed)
    bN, bK = tile
    W = weights(rng, N, K)
    z = map_bands(rng, N // bN, K // bK, 0.30)
    X = acts_heavy_tail(rng, M, K)
    return dict(W=W, zmap=z, X=X, bN=bN, bK=bK, name=f"qwen4b.{name}.M{M}")


def dense8b_maps(seed: int = 4000, tile=TILE) -> list[list[np.ndarray]]:
    """Per layer: f8 ~ U(0.15, 0.45); the layer's tiles are pooled and
    round(f8 * T_layer) of them are made INT8 uniformly."""
    rng = np.random.default_rng(seed)
    bN, bK = tile
    maps = []
    for _ in range(DENSE8B_LAYERS):
        f8 = rng.uniform(0.15, 0.45)
        geo = [(N // bN, K // bK) for _, N, K in DENSE8B]
        T = sum(R * C for R, C in geo)
        flat = np.full(T, 4, dtype=np.int8)
        flat[rng.permutation(T)[:count_from_fraction(f8, T)]] = 8
        layer, o = [], 0
        for R, C in geo:
            layer.append(flat[o:o + R * C].reshape(R, C))
            o += R * C
        maps.append(layer)
    return maps


def qwen14b_maps(seed: int = 5000, tile=TILE) -> list[list[np.ndarray]]:
    """Model-wide 30% INT8, o/down tiles weighted 3x."""
    rng = np.random.default_rng(seed)
    bN, bK = tile
    geoms = []
    for _ in range(QWEN14B_LAYERS):
        for name, N, K in QWEN14B:
            geoms.append((N // bN, K // bK, 3.0 if name in ("o", "down") else 1.0))
    flat = map_model_weighted(rng, geoms, 0.30)
    return [flat[4 * l:4 * l + 4] for l in range(QWEN14B_LAYERS)]


def device_weights(N: int, K: int, seed: int, device="cuda", std: float = 0.02):
    """W ~ N(0, std) generated on the device with a seeded torch generator
    (the large model-wide workloads do not pass through host memory)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32).mul_(std)


def device_acts_outliers(M: int, K: int, seed: int, device="cuda", frac: float = 0.01, mult: float = 30.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    n = max(1, int(round(frac * K)))
    ch = torch.randperm(K, generator=g, device=device)[:n]
    X[:, ch] *= mult
    return X


def device_acts_heavy_tail(M: int, K: int, seed: int, device="cuda", frac: float = 0.05, nu: float = 3.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    n = max(1, int(round(frac * K)))
    ch = torch.randperm(K, generator=g, device=device)[:n]
    # Student-t(nu), integer nu: Z / sqrt(chi2_nu / nu), chi2_nu = sum of nu squared normals
    k = int(nu)
    z = torch.randn((M, n), generator=g, device=device, dtype=torch.float32)
    chi2 = torch.randn((k, M, n), generator=g, device=device, dtype=torch.float32).square().sum(0)
    X[:, ch] = z / torch.sqrt(chi2 / k)
    return X
