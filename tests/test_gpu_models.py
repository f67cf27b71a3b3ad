"""GPU parity on the two whole-model workloads, through the C ABI.

  8B-class dense model (hidden 4096, 32 q / 8 kv heads x 128, FFN 14336,
  36 layers; per-layer INT8 fraction ~ U(0.15, 0.45)): all 144 projections
  packed and resident in HBM, one decode step over all of them at
  M = 1, 8, 32 and 64 tokens.
  Qwen3-14B-shaped model (hidden 5120, 40 q / 8 kv heads x 128, FFN 17408,
  40 layers; model-wide 30% INT8 weighted 3x toward o/down): all 160
  projections packed; M = 8192 prefill chunks of the 64K-token prompt, then
  one batch-32 decode step from the same packed weights.

The GPU runs every call at full size in the benchmarked launch shapes.  The
oracle checks samples: layers {first, middle, last}; per projection six
tile rows (the first, the last and four seeded), i.e. 384 output channels
over the full K; all decode tokens; for prefill 24 token rows (block
boundaries and seeded).  On the samples, packed bytes, labels, row offsets,
activation codes and scales, and INT32 tile products are bit-exact, and
outputs meet the bar stated in tests/parity.py.
"""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from mixed_precision_int_amd.model import pack_model, tile_row_slices
from oracle import aq_oracle as O
from tests.parity import assert_output_close, say
from workloads import gen

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

BK = gen.TILE[1]


def _weights(config):
    return lambda l, name, N, K: gen.device_weights(N, K, gen.seed_for(config, l, name))


def _sampled_layers(L):
    return (0, L // 2, L - 1)


def _sample_tile_rows(R, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, R - 1), 4, replace=False)
    return np.unique(np.concatenate([[0, R - 1], mid]))


def _channels(tile_rows):
    return np.concatenate([np.arange(64 * r, 64 * r + 64) for r in tile_rows])


_SAMPLES = {}


def sample(config, l, name, N, K, zmap):
    """The oracle view of a projection's sampled tile rows, built once."""
    key = (config, l, name)
    if key not in _SAMPLES:
        _SAMPLES[key] = Sample(config, l, name, N, K, zmap)
    return _SAMPLES[key]


class Sample:
    """Oracle view of sampled tile rows of one packed projection."""

    def __init__(self, config, l, name, N, K, zmap):
        self.name = f"cfg{config}.L{l}.{name}"
        self.zmap = np.asarray(zmap)
        self.tile_rows = _sample_tile_rows(N // 64, gen.seed_for(config, l, name))
        self.cols = _channels(self.tile_rows)
        W = gen.device_weights(N, K, gen.seed_for(config, l, name))
        W_sub = W[torch.from_numpy(self.cols).cuda()].cpu().numpy()
        del W
        z_sub = self.zmap[self.tile_rows]
        self.codes, self.sW = O.quant_weights(W_sub, z_sub, 64, BK)
        self.pk = O.pack(self.codes, self.sW, z_sub, 64, BK)

    def check_pack(self, pw):
        got = tile_row_slices(pw, self.tile_rows)
        assert np.array_equal(got["labels"], O.labels_from_map(self.zmap)), self.name
        assert np.array_equal(got["row_off4"], O.row_offsets(self.zmap, 4)), self.name
        assert np.array_equal(got["row_off8"], O.row_offsets(self.zmap, 8)), self.name
        for k in ("w4", "w8"):
            assert np.array_equal(got[k], self.pk[k]), f"{self.name}: {k} bytes differ"
        for k in ("s4", "s8"):
            assert np.array_equal(got[k].view(np.uint32), self.pk[k].view(np.uint32)), \
                f"{self.name}: {k} bits differ"

    def check_call(self, pw, X_rows, qx_d, sx_d, Y_d, token_rows, phase, tag, full_products=False):
        """Codes, scales, tile products and outputs of the sampled rows.
        full_products: the tile products come from a call over all of
        qx_d's rows (the route and launch shape of the timed call), gathered
        at the sampled rows on the device; otherwise from a call over the
        gathered rows."""
        rows_d = torch.from_numpy(np.asarray(token_rows)).cuda()
        qx_ref, sx_ref = O.quant_act(X_rows)
        qx_g = qx_d.index_select(0, rows_d).contiguous()
        sx_g = sx_d.index_select(0, rows_d).contiguous()
        assert np.array_equal(qx_g.cpu().numpy().astype(np.int64), qx_ref), f"{self.name}/{tag}: qx"
        assert np.array_equal(sx_g.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32)), \
            f"{self.name}/{tag}: sx bits"
        P_ref = O.tile_partials(qx_ref, self.codes, BK)
        cols_d = torch.from_numpy(self.cols).cuda()
        if full_products:
            P = aq.aq_linear_tile_partials(pw, qx_d, phase)
            P_g = P.index_select(0, rows_d).index_select(1, cols_d).cpu().numpy().astype(np.int64)
        else:
            P = aq.aq_linear_tile_partials(pw, qx_g, phase)
            P_g = P.index_select(1, cols_d).cpu().numpy().astype(np.int64)
        del P
        bad = np.argwhere(P_g != P_ref)
        assert bad.size == 0, f"{self.name}/{tag}: {len(bad)} tile products differ, first {bad[:4].tolist()}"
        y = O.linear_from_partials(P_ref, sx_ref, self.sW)
        c = O.abs_contrib(P_ref, sx_ref, self.sW)
        Y_g = Y_d.index_select(0, rows_d).index_select(1, cols_d).cpu().numpy()
        assert_output_close(Y_g, y, c, f"{self.name}/{tag}")


# ------------------------------------------------------------ 8B-class model

@pytest.fixture(scope="module")
def dense8b():
    maps = gen.dense8b_maps()
    say(f"[dense8b] packing {gen.DENSE8B_LAYERS} layers x {len(gen.DENSE8B)} projections")
    model = pack_model(gen.DENSE8B, maps, _weights(4),
                       progress=lambda l: (l % 6 == 5) and say(f"  packed layer {l}"))
    torch.cuda.synchronize()
    say(f"  packed model {model.nbytes() / 1e9:.3f} GB resident")
    yield model, maps
    del model
    torch.cuda.empty_cache()


def test_dense8b_pack_sampled_layers(dense8b):
    model, maps = dense8b
    for l in _sampled_layers(gen.DENSE8B_LAYERS):
        for p, (name, N, K) in enumerate(gen.DENSE8B):
            s = sample(4, l, name, N, K, maps[l][p])
            s.check_pack(model.layers[l][name])
            say(f"  {s.name}: pack bit-exact on tile rows {s.tile_rows.tolist()}")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_dense8b_decode_step(dense8b, M):
    """One decode step through all 144 projections; sampled layers checked."""
    model, maps = dense8b
    check = set(_sampled_layers(gen.DENSE8B_LAYERS))
    samples = {}
    for l, name, pw in model:
        X = gen.device_acts_outliers(M, pw.K, gen.act_seed(4, l, name, M))
        qx, sx = aq.aq_quant_act(X)
        Y = aq.aq_linear_decode(pw, qx, sx)
        if l in check:
            samples[(l, name)] = (X, qx, sx, Y)
    torch.cuda.synchronize()
    say(f"[dense8b] decode step M={M}: {len(model.layers) * len(model.geometry)} calls done")
    for (l, name), (X, qx, sx, Y) in samples.items():
        p = [g[0] for g in gen.DENSE8B].index(name)
        _, N, K = gen.DENSE8B[p]
        s = sample(4, l, name, N, K, maps[l][p])
        s.check_call(model.layers[l][name], X.cpu().numpy(), qx, sx, Y, np.arange(M),
                     aq.AQ_PHASE_DECODE, f"decode.M{M}")


# ------------------------------------------------------------ Qwen3-14B-shaped model

@pytest.fixture(scope="module")
def qwen14b():
    maps = gen.qwen14b_maps()
    say(f"[qwen14b] packing {gen.QWEN14B_LAYERS} layers x {len(gen.QWEN14B)} projections")
    model = pack_model(gen.QWEN14B, maps, _weights(5),
                       progress=lambda l: (l % 8 == 7) and say(f"  packed layer {l}"))
    torch.cuda.synchronize()
    t8 = sum(int(np.sum(z == 8)) for layer in maps for z in layer)
    t = sum(z.size for layer in maps for z in layer)
    say(f"  packed model {model.nbytes() / 1e9:.3f} GB resident, INT8 tiles {t8}/{t} = {t8 / t:.4f}")
    yield model, maps
    del model
    torch.cuda.empty_cache()


def test_qwen14b_map_budget_and_pack(qwen14b):
    """The model-wide budget is round(0.30 T) INT8 tiles, skewed toward o/down;
    sampled layers pack bit-exact."""
    model, maps = qwen14b
    t = sum(z.size for layer in maps for z in layer)
    t8 = sum(int(np.sum(z == 8)) for layer in maps for z in layer)
    assert t8 == O.int8_tile_count(0.30, t)
    frac = {name: np.mean([np.mean(maps[l][p] == 8) for l in range(len(maps))])
            for p, (name, _, _) in enumerate(gen.QWEN14B)}
    say(f"  INT8 fraction per projection: {frac}")
    assert min(frac["o"], frac["down"]) > max(frac["qkv"], frac["gate_up"])
    for l in _sampled_layers(gen.QWEN14B_LAYERS):
        for p, (name, N, K) in enumerate(gen.QWEN14B):
            s = sample(5, l, name, N, K, maps[l][p])
            s.check_pack(model.layers[l][name])
            say(f"  {s.name}: pack bit-exact on tile rows {s.tile_rows.tolist()}")


@pytest.mark.parametrize("chunk", [0, 7])
def test_qwen14b_prefill_chunk(qwen14b, chunk):
    """M = 8192 prefill chunks (the first and the last of the 64K prompt)
    through every projection of the sampled layers."""
    model, maps = qwen14b
    rng = np.random.default_rng(500 + chunk)
    M = 8192
    rows = np.unique(np.concatenate([[0, 127, 128, 4095, 8191], rng.choice(M, 19, replace=False)]))
    for l in _sampled_layers(gen.QWEN14B_LAYERS):
        for p, (name, N, K) in enumerate(gen.QWEN14B):
            pw = model.layers[l][name]
            X = gen.device_acts_heavy_tail(M, K, gen.act_seed(5, l, name, chunk))
            qx, sx = aq.aq_quant_act(X)
            Y = aq.aq_linear_prefill(pw, qx, sx)
            X_rows = X.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
            del X
            s = sample(5, l, name, N, K, maps[l][p])
            # the o projection of the first chunk of layer 0 also compares the
            # products of the whole 8192-row call (long route, 6.7 GB of INT32)
            full = chunk == 0 and l == 0 and name == "o"
            s.check_call(pw, X_rows, qx, sx, Y, rows, aq.AQ_PHASE_PREFILL, f"prefill.chunk{chunk}",
                         full_products=full)
            del qx, sx, Y


def test_qwen14b_decode_batch32(qwen14b):
    """One batch-32 decode step through all 160 projections after prefill."""
    model, maps = qwen14b
    check = set(_sampled_layers(gen.QWEN14B_LAYERS))
    samples = {}
    for l, name, pw in model:
        X = gen.device_acts_outliers(32, pw.K, gen.act_seed(5, l, name, 100))
        qx, sx = aq.aq_quant_act(X)
        Y = aq.aq_linear_decode(pw, qx, sx)
        if l in check:
            samples[(l, name)] = (X, qx, sx, Y)
    torch.cuda.synchronize()
    say(f"[qwen14b] decode step M=32: {len(model.layers) * len(model.geometry)} calls done")
    for (l, name), (X, qx, sx, Y) in samples.items():
        p = [g[0] for g in gen.QWEN14B].index(name)
        _, N, K = gen.QWEN14B[p]
        s = sample(5, l, name, N, K, maps[l][p])
        s.check_call(model.layers[l][name], X.cpu().numpy(), qx, sx, Y, np.arange(32),
                     aq.AQ_PHASE_DECODE, "decode.M32")
