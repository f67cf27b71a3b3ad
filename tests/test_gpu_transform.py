"""GPU parity of the tile-aligned block transforms (App. B.1, eq. 4) through
the C ABI, against the oracle.  X~ = X V and W~ = U W V feed quantizers, so
both follow one fixed FP32 evaluation order and must match the oracle to
the last bit; Y = Y~ U is compared with the oracle's FP64 product within the
FP32 error of six butterfly stages: per 64-block, |error|_2 <= 3e-6 |y~|_2
(6 roundings of relative size 2^-24 on values whose 2-norm the orthonormal
stages preserve, with margin).  The transformed linear runs the untouched
decode / prefill kernels on transformed operands; its codes, scales and
outputs meet the bar of the untransformed path."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import assert_output_close, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu

TABLES = gen.transform_tables()


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def assert_bits_equal(got, ref, name):
    bad = np.argwhere(bits(got) != bits(ref))
    assert bad.size == 0, f"{name}: {len(bad)} values differ, first {bad[:4].tolist()}"


def assert_blocks_close(got, ref, name, rel=3e-6, src=None):
    """Per 64-block, |got - ref|_2 <= rel |src|_2 + 2^-23 |ref|_2 (src: the
    block before the transform, default ref; the second term covers one
    final FP32 rounding, such as a bias add)."""
    M, N = ref.shape
    g = np.asarray(got, np.float64).reshape(M, N // 64, 64)
    r = np.asarray(ref, np.float64).reshape(M, N // 64, 64)
    s0 = r if src is None else np.asarray(src, np.float64).reshape(M, N // 64, 64)
    err = np.linalg.norm(g - r, axis=-1)
    bound = rel * np.linalg.norm(s0, axis=-1) + 2.0 ** -23 * np.linalg.norm(r, axis=-1) + 1e-30
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{name}: {len(bad)} blocks off, first {bad[:4].tolist()}"


def every_seed(rng, n):
    """n seeds covering all of -1 .. 6 when n >= 8, the rest drawn."""
    s = gen.transform_seeds(rng, n)
    s[:min(n, 8)] = np.arange(-1, 7)[:min(n, 8)]
    return s


@pytest.mark.parametrize("M,K", [(1, 64), (5, 512), (33, 1088), (64, 4096), (3, 14336)])
def test_transform_rows_bit_exact(M, K):
    """X~ = X V over every seed, ragged workgroup tails (1088 = 17 blocks)."""
    rng = np.random.default_rng(7 * M + K)
    X = gen.acts_outliers(rng, M, K, max(1, K // 200), 25.0)
    vs = every_seed(rng, K // 64)
    say(f"  transform_rows M={M} K={K}")
    Xt = aq.aq_transform_rows(to_dev(X), vs, TABLES)
    torch.cuda.synchronize()
    assert_bits_equal(Xt.cpu().numpy(), O.transform_rows(X, vs, TABLES), f"rows M{M} K{K}")
    # in place gives the same bits
    Xd = to_dev(X)
    aq.aq_transform_rows(Xd, vs, TABLES, out=Xd)
    torch.cuda.synchronize()
    assert_bits_equal(Xd.cpu().numpy(), Xt.cpu().numpy(), f"rows in place M{M} K{K}")


@pytest.mark.parametrize("N,K", [(64, 64), (192, 320), (512, 1024), (4096, 4096)])
def test_transform_weights_bit_exact(N, K):
    """W~ = U W V: row blocks, then the columns of every output tile row."""
    rng = np.random.default_rng(N + 3 * K)
    W = gen.weights(rng, N, K)
    us, vs = every_seed(rng, N // 64), every_seed(rng, K // 64)
    say(f"  transform_weights N={N} K={K}")
    Wt = aq.aq_transform_weights(to_dev(W), us, vs, TABLES)
    torch.cuda.synchronize()
    assert_bits_equal(Wt.cpu().numpy(), O.transform_weights(W, us, vs, TABLES), f"weights N{N} K{K}")


@pytest.mark.parametrize("M,N,bias", [(1, 64, False), (4, 576, True), (37, 4096, True), (1024, 1024, False)])
def test_transform_out_close(M, N, bias):
    """Y = Y~ U (+ bias) against the FP64 product, in place and out of place."""
    rng = np.random.default_rng(11 * M + N)
    Yt = (rng.standard_normal((M, N)) * rng.uniform(0.1, 30.0, size=(M, 1))).astype(np.float32)
    us = every_seed(rng, N // 64)
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    ref = O.transform_out(Yt, us, TABLES) + (0.0 if b is None else b.astype(np.float64)[None, :])
    say(f"  transform_out M={M} N={N} bias={bias}")
    bd = None if b is None else to_dev(b)
    Y = aq.aq_transform_out(to_dev(Yt), us, TABLES, bias=bd)
    Yd = to_dev(Yt)
    aq.aq_transform_out(Yd, us, TABLES, bias=bd, out=Yd)
    torch.cuda.synchronize()
    assert_blocks_close(Y.cpu().numpy(), ref, f"out M{M} N{N}", src=Yt)
    assert_bits_equal(Yd.cpu().numpy(), Y.cpu().numpy(), f"out in place M{M} N{N}")


@pytest.mark.parametrize("M,K", [(1, 64), (5, 3072), (33, 1088), (255, 4096), (7, 4160), (300, 9728), (2, 40768),
                                 (256, 2560)])
def test_quant_act_transformed_bit_exact(M, K):
    """X V and the per-token quantizer in one pass: codes and scales equal the
    oracle's quantizer applied to the oracle's X V, on every layout (fewer
    than 256 rows of at most 64 blocks: lane by element; other rows: the quad
    layout on 1024 or 256 threads) and the longest row the on-chip staging
    takes; a zero row keeps the 1e-12 floor."""
    rng = np.random.default_rng(13 * M + K)
    X = gen.acts_outliers(rng, M, K, max(1, K // 100), 30.0)
    X[0, :] = 0.0
    vs = every_seed(rng, K // 64)
    qx_r, sx_r = O.quant_act(O.transform_rows(X, vs, TABLES))
    say(f"  quant_act_transformed M={M} K={K}")
    qx, sx = aq.aq_quant_act_transformed(to_dev(X), vs, TABLES)
    torch.cuda.synchronize()
    assert np.array_equal(qx.cpu().numpy().astype(np.int64), qx_r), f"M{M} K{K}: codes differ"
    assert_bits_equal(sx.cpu().numpy(), sx_r, f"M{M} K{K}: scales")


def test_quant_act_transformed_bad_seed():
    """A seed outside -1 .. 6 gives every row a NaN scale."""
    X = np.ones((3, 128), np.float32)
    _, sx = aq.aq_quant_act_transformed(to_dev(X), np.array([0, 8], np.int8), TABLES)
    assert np.isnan(sx.cpu().numpy()).all()


def test_transform_round_trip():
    """Phi_s applied after Phi_s^T returns the input up to FP32 rounding (the
    transforms are orthogonal)."""
    rng = np.random.default_rng(5)
    X = gen.acts_outliers(rng, 8, 1024, 10, 20.0)
    s = every_seed(rng, 16)
    back = aq.aq_transform_out(aq.aq_transform_rows(to_dev(X), s, TABLES), s, TABLES)
    torch.cuda.synchronize()
    assert_blocks_close(back.cpu().numpy(), X.astype(np.float64), "round trip", rel=6e-6)


def test_transform_bad_seed_gives_nan():
    """A seed outside -1 .. 6 is not a transform: its block comes out NaN and
    the others are untouched."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal((3, 256)).astype(np.float32)
    s = np.array([0, 7, -1, -2], np.int8)
    Xt = aq.aq_transform_rows(to_dev(X), s, TABLES).cpu().numpy()
    assert np.isnan(Xt[:, 64:128]).all() and np.isnan(Xt[:, 192:]).all()
    ok = np.array([0, -1, -1, -1], np.int8)
    ref = O.transform_rows(X, ok, TABLES)
    assert_bits_equal(Xt[:, :64], ref[:, :64], "seed 0 block")
    assert_bits_equal(Xt[:, 128:192], ref[:, 128:192], "identity block")
    W = gen.weights(rng, 128, 128)
    Wt = aq.aq_transform_weights(to_dev(W), np.array([1, 9], np.int8), np.array([2, 3], np.int8),
                                 TABLES).cpu().numpy()
    assert not np.isnan(Wt[:64]).any() and np.isnan(Wt[64:]).all()


@pytest.mark.parametrize("N,K,bK,M", [(256, 1024, 128, 1), (192, 768, 128, 16), (256, 512, 64, 37),
                                      (320, 2560, 128, 1030)])
def test_transformed_linear(N, K, bK, M):
    """The transformed layer end to end (App. B.1): W~ = U W V packed with the
    App. E map, X~ = X V quantized per token, the decode (or long prefill)
    kernels give Y~, and Y = Y~ U.  Every integer stage bit-exact with the
    oracle on the oracle's own transformed operands; Y~ within the linear's
    bar; Y within the transform's bound of the oracle's Y~ U of the GPU Y~;
    and Y close to X W^T + bias where quantization error allows
    (orthogonality)."""
    rng = np.random.default_rng(N + K + M)
    W = gen.weights(rng, N, K)
    X = gen.acts_outliers(rng, M, K, max(1, K // 100), 25.0)
    R, C = N // 64, K // bK
    z = gen.map_uniform(rng, R, C, 0.35)
    us, vs = every_seed(rng, R), every_seed(rng, K // 64)
    b = rng.standard_normal(N).astype(np.float32)
    name = f"transformed{N}x{K}/bK{bK}/M{M}"
    say(f"[{name}]")
    # oracle
    Wt_r = O.transform_weights(W, us, vs, TABLES)
    Xt_r = O.transform_rows(X, vs, TABLES)
    codes, sW = O.quant_weights(Wt_r, z, 64, bK)
    qx_r, sx_r = O.quant_act(Xt_r)
    P_r = O.tile_partials(qx_r, codes, bK)
    yt_r = O.linear_from_partials(P_r, sx_r, sW)
    # HIP path
    Wt = aq.aq_transform_weights(to_dev(W), us, vs, TABLES)
    pw = aq.aq_pack_weights(Wt, aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    qx, sx = aq.aq_quant_act_transformed(to_dev(X), vs, TABLES)
    Yt = aq.aq_linear_decode(pw, qx, sx) if M < 1024 else aq.aq_linear_prefill(pw, qx, sx)
    Y = aq.aq_transform_out(Yt, us, TABLES, bias=to_dev(b))
    torch.cuda.synchronize()
    assert_bits_equal(Wt.cpu().numpy(), Wt_r, f"{name}: W~")
    assert np.array_equal(qx.cpu().numpy().astype(np.int64), qx_r), f"{name}: codes differ"
    assert_bits_equal(sx.cpu().numpy(), sx_r, f"{name}: activation scales")
    Yt_h = Yt.cpu().numpy()
    assert_output_close(Yt_h, yt_r, O.abs_contrib(P_r, sx_r, sW), f"{name}: Y~")
    assert_blocks_close(Y.cpu().numpy(), O.transform_out(Yt_h, us, TABLES) + b[None, :], f"{name}: Y", src=Yt_h)
    # U and V orthogonal: Y~ U approximates X W^T up to the quantization error
    y_fp = X.astype(np.float64) @ W.astype(np.float64).T + b[None, :]
    rel = np.linalg.norm(Y.cpu().numpy() - y_fp) / np.linalg.norm(y_fp)
    assert rel < 0.1, f"{name}: transformed layer far from X W^T ({rel:.3g})"


@pytest.mark.parametrize("proj", ["qkv", "down"])
def test_transforms_full_prefill_size_sampled(proj):
    """Full Qwen3-4B-shaped prefill size (M = 2048), in the launch shapes the
    transform benchmark times: the one-pass quantizer's codes and scales on
    sampled token rows, bit-exact with the oracle's quantizer of the
    oracle's X V, and Y~ U (+ bias) of the full [2048, N] output on the same
    rows within the transform bound."""
    d = gen.qwen4b_prefill(proj, 2048)
    X = d["X"]
    M, K = X.shape
    N = d["W"].shape[0]
    rng = np.random.default_rng(K + N)
    vs, us = every_seed(rng, K // 64), every_seed(rng, N // 64)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], rng.choice(M, 11, replace=False)]))
    say(f"  full-size transforms {proj} M={M} K={K} N={N}, rows {rows.tolist()}")
    qx, sx = aq.aq_quant_act_transformed(to_dev(X), vs, TABLES)
    Yt = (rng.standard_normal((M, N)) * 4.0).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    Y = aq.aq_transform_out(to_dev(Yt), us, TABLES, bias=to_dev(b))
    torch.cuda.synchronize()
    qx_r, sx_r = O.quant_act(O.transform_rows(X[rows], vs, TABLES))
    assert np.array_equal(qx.cpu().numpy()[rows].astype(np.int64), qx_r), f"{proj}: codes differ"
    assert_bits_equal(sx.cpu().numpy()[rows], sx_r, f"{proj}: scales")
    ref = O.transform_out(Yt[rows], us, TABLES) + b.astype(np.float64)[None, :]
    assert_blocks_close(Y.cpu().numpy()[rows], ref, f"{proj}: Y", src=Yt[rows])


@pytest.mark.parametrize("N,K,bK,M,bias", [(256, 1024, 128, 1030, True), (320, 2560, 128, 2048, False),
                                           (256, 640, 64, 1040, True), (192, 768, 128, 100, True),
                                           (256, 640, 64, 300, False), (6144, 2560, 128, 2048, True),
                                           (8192, 1024, 128, 1040, True), (3072, 8192, 128, 40, True),
                                           (512, 3072, 128, 9, False)])
def test_prefill_transformed(N, K, bK, M, bias):
    """Y = Y~ U + bias with U applied inside the GEMMs' epilogue (M >= 1024:
    the 256 x 128 kernel, or the persistent 256 x 256 one for the wide
    shapes, 6144 x 2560 and 8192 x 1024 with a ragged last M-block; shorter
    prompts: the 32 x 32 MFMA kernel at b_K = 128 and 64; up to 64 rows the
    decode kernels, with tile rows handed over through the workspace at
    3072 x 8192, M = 40): within FP32 rounding of
    aq_linear_prefill followed by aq_transform_out (per 64-block,
    |difference|_2 <= 1e-5 |y~|_2: the token scale is applied after U instead
    of before), and every seed value on some tile row."""
    rng = np.random.default_rng(N + K + M)
    W = gen.weights(rng, N, K)
    R, C = N // 64, K // bK
    z = gen.map_uniform(rng, R, C, 0.35)
    X = gen.acts_heavy_tail(rng, M, K)
    us = every_seed(rng, R)
    b = to_dev(rng.standard_normal(N).astype(np.float32)) if bias else None
    say(f"  prefill_transformed {N}x{K}/bK{bK}/M{M}")
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    qx, sx = aq.aq_quant_act(to_dev(X))
    Yt = aq.aq_linear_prefill(pw, qx, sx)
    ref = aq.aq_transform_out(Yt, us, TABLES, bias=b)
    Y = aq.aq_linear_prefill_transformed(pw, qx, sx, us, TABLES, bias=b)
    Y2 = aq.aq_linear_prefill_transformed(pw, qx, sx, us, TABLES, bias=b)
    torch.cuda.synchronize()
    assert_blocks_close(Y.cpu().numpy(), ref.cpu().numpy().astype(np.float64), f"{N}x{K}/M{M}", rel=1e-5,
                        src=Yt.cpu().numpy())
    # every wave of every launch takes the same sign tables: repeated calls agree bit for bit
    assert torch.equal(Y, Y2), f"{N}x{K}/M{M}: repeated calls differ"


@pytest.mark.parametrize("N,K,M", [(320, 2560, 300), (320, 2560, 1030), (6144, 2560, 2048)])
def test_prefill_transformed_against_oracle(N, K, M):
    """The fused route end to end on sampled rows: W~ = U W V packed, X~
    quantized in one pass, Y = Y~ U + bias from the GEMM epilogue, against the
    oracle's transformed layer.  6144 x 2560 at M = 2048 is the Qwen3-4B qkv
    shape at the benchmarked prompt length: 96 tile rows (both tile-row
    waves of every 256 x 128 block, every seed value) and sampled token rows
    in each of the four 64-row waves of a block, in first, middle and last
    blocks."""
    rng = np.random.default_rng(17 + N)
    W = gen.weights(rng, N, K)
    X = gen.acts_outliers(rng, M, K, 25, 25.0)
    z = gen.map_uniform(rng, N // 64, K // 128, 0.35)
    us, vs = every_seed(rng, N // 64), every_seed(rng, K // 64)
    b = rng.standard_normal(N).astype(np.float32)
    if M < 2048:
        rows = np.array([0, 1, 63, 64, 255, M - 1])
    else:
        rows = np.unique(np.concatenate([[0, 63, 64, 127, 128, 191, 192, 255, 1024, 1100, 1170, 1250, M - 1],
                                         rng.choice(M, 7, replace=False)]))
    say(f"  fused transformed prefill {N}x{K}/M{M} against the oracle, rows {rows.tolist()}")
    Wt_r = O.transform_weights(W, us, vs, TABLES)
    codes, sW = O.quant_weights(Wt_r, z, 64, 128)
    qx_r, sx_r = O.quant_act(O.transform_rows(X[rows], vs, TABLES))
    P = O.tile_partials(qx_r, codes, 128)
    y_ref = O.transform_out(O.linear_from_partials(P, sx_r, sW), us, TABLES) + b.astype(np.float64)[None, :]
    pw = aq.aq_pack_weights(aq.aq_transform_weights(to_dev(W), us, vs, TABLES),
                            aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
    qx, sx = aq.aq_quant_act_transformed(to_dev(X), vs, TABLES)
    Y = aq.aq_linear_prefill_transformed(pw, qx, sx, us, TABLES, bias=to_dev(b))
    torch.cuda.synchronize()
    yt_norm = O.linear_from_partials(P, sx_r, sW)
    assert_blocks_close(Y.cpu().numpy()[rows], y_ref, "fused transformed prefill", rel=1e-4, src=yt_norm)


def test_prefill_transformed_bad_seed():
    """A seed outside -1 .. 6 turns its tile row's outputs NaN; the others
    are finite."""
    rng = np.random.default_rng(3)
    W = gen.weights(rng, 128, 256)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(np.full((2, 2), 4, np.uint8)), 64, 128)
    qx, sx = aq.aq_quant_act(to_dev(gen.acts_heavy_tail(rng, 1024, 256)))
    Y = aq.aq_linear_prefill_transformed(pw, qx, sx, np.array([0, 9], np.int8), TABLES).cpu().numpy()
    assert np.isfinite(Y[:, :64]).all() and np.isnan(Y[:, 64:]).all()


# Decode with U in its epilogue.  The Llama-3.2-3B-shaped projections cover
# every way the planner lays out a tile row: one workgroup per tile row
# (gate_up, 4 row groups per workgroup), row groups spread over 2 or 4
# workgroups (qkv, o, down at M <= 32), and column chunks (down at M = 64,
# whose activations do not fit on chip), at M in the per-wave-slice (<= 4),
# shared-staging and multi-chunk (> 64 tokens) routes.
DECODE_XF_CASES = [("qkv", 5120, 3072, 1), ("o", 3072, 3072, 4), ("gate_up", 16384, 3072, 16),
                   ("down", 3072, 8192, 16), ("down", 3072, 8192, 64), ("o", 3072, 3072, 33),
                   ("qkv", 5120, 3072, 100), ("small64", 256, 640, 5)]


def _decode_xf_setup(name, N, K, M, seed):
    bK = 64 if name == "small64" else 128
    rng = np.random.default_rng(seed)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // bK, 0.25)
    X = gen.acts_outliers(rng, M, K, max(1, K // 100), 25.0)
    us = every_seed(rng, N // 64)
    b = rng.standard_normal(N).astype(np.float32)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    qx, sx = aq.aq_quant_act(to_dev(X))
    return pw, qx, sx, us, to_dev(b)


@pytest.mark.parametrize("name,N,K,M", DECODE_XF_CASES)
def test_decode_transformed_bit_exact(name, N, K, M):
    """aq_linear_decode_transformed is bit for bit aq_linear_decode (no bias)
    with the same split followed by aq_transform_out (bias), at every fixed
    split (which moves the tile row between one workgroup and several), with
    and without a bias.  The adaptive call takes either the plain decode's
    adaptive split or 4 waves per row group (the tile row in one workgroup),
    and matches that call bit for bit."""
    pw, qx, sx, us, b = _decode_xf_setup(name, N, K, M, N + K + M)
    Wv = 16  # waves per decode workgroup
    for bias in (b, None):
        refs = {}
        for split in (Wv, Wv // 2, Wv // 4):
            say(f"  decode_transformed {name} {N}x{K} M={M} split={split} bias={bias is not None}")
            Yt = aq.aq_linear_decode(pw, qx, sx, split=split)
            ref = aq.aq_transform_out(Yt, us, TABLES, bias=bias).cpu().numpy()
            Y = aq.aq_linear_decode_transformed(pw, qx, sx, us, TABLES, bias=bias, split=split)
            torch.cuda.synchronize()
            assert_bits_equal(Y.cpu().numpy(), ref, f"{name}/M{M}/split{split}")
            refs[split] = ref
        Y0 = aq.aq_linear_decode_transformed(pw, qx, sx, us, TABLES, bias=bias).cpu().numpy()
        cands = (aq.aq_decode_split(pw, M), Wv // 4)
        assert any(np.array_equal(bits(Y0), bits(refs[c])) for c in cands), \
            f"{name}/M{M}: the adaptive call matches neither split {cands}"


def test_decode_transformed_against_oracle():
    """The fused decode end to end against the oracle's transformed layer:
    W~ = U W V packed, X~ = X V quantized in one pass, Y = Y~ U + bias from the
    decode epilogue, on the Llama-3.2-3B-shaped o projection at M = 4 (row
    groups of a tile row in four workgroups) and a 64 x 64-tile case."""
    for N, K, bK, M in ((3072, 3072, 128, 4), (256, 640, 64, 7)):
        rng = np.random.default_rng(5 + N + M)
        W = gen.weights(rng, N, K)
        X = gen.acts_outliers(rng, M, K, max(1, K // 100), 25.0)
        z = gen.map_uniform(rng, N // 64, K // bK, 0.3)
        us, vs = every_seed(rng, N // 64), every_seed(rng, K // 64)
        b = rng.standard_normal(N).astype(np.float32)
        say(f"  fused transformed decode {N}x{K}/bK{bK}/M{M} against the oracle")
        Wt_r = O.transform_weights(W, us, vs, TABLES)
        codes, sW = O.quant_weights(Wt_r, z, 64, bK)
        qx_r, sx_r = O.quant_act(O.transform_rows(X, vs, TABLES))
        P = O.tile_partials(qx_r, codes, bK)
        yt = O.linear_from_partials(P, sx_r, sW)
        y_ref = O.transform_out(yt, us, TABLES) + b.astype(np.float64)[None, :]
        pw = aq.aq_pack_weights(aq.aq_transform_weights(to_dev(W), us, vs, TABLES),
                                aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
        qx, sx = aq.aq_quant_act_transformed(to_dev(X), vs, TABLES)
        Y = aq.aq_linear_decode_transformed(pw, qx, sx, us, TABLES, bias=to_dev(b))
        torch.cuda.synchronize()
        assert np.array_equal(qx.cpu().numpy().astype(np.int64), qx_r), "codes differ"
        assert_blocks_close(Y.cpu().numpy(), y_ref, f"fused transformed decode {N}x{K}", rel=1e-4, src=yt)


def test_decode_transformed_calls_in_a_row():
    """Calls that hand tile rows over leave their arrival counters at zero:
    transformed and plain decode calls of different sizes on one workspace,
    one after another, each equal to its reference."""
    pw, qx, sx, us, b = _decode_xf_setup("o", 3072, 3072, 64, 11)
    need = max(aq.aq_workspace_bytes(pw, M, ph, 16) for M in (1, 16, 64)
               for ph in (aq.AQ_PHASE_DECODE, aq.AQ_PHASE_DECODE_TRANSFORMED))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for M in (16, 1, 64, 16):
        sp = 16  # one row group per workgroup: every tile row handed over
        say(f"  decode_transformed in a row: M={M} split={sp}")
        Yt = aq.aq_linear_decode(pw, qx[:M], sx[:M], split=sp, ws=ws)
        ref = aq.aq_transform_out(Yt, us, TABLES, bias=b)
        Y = aq.aq_linear_decode_transformed(pw, qx[:M], sx[:M], us, TABLES, bias=b, split=sp, ws=ws)
        torch.cuda.synchronize()
        assert_bits_equal(Y.cpu().numpy(), ref.cpu().numpy(), f"in a row M={M}")
    assert int(ws[:4 * 65536].view(torch.int32).abs().sum()) == 0, "arrival counters left set"


def test_decode_transformed_bad_seed():
    """A seed outside -1 .. 6 turns its tile row's outputs NaN; the others
    are finite."""
    pw, qx, sx, _, _ = _decode_xf_setup("small64", 256, 640, 3, 2)
    Y = aq.aq_linear_decode_transformed(pw, qx, sx, np.array([0, 9, -1, 6], np.int8), TABLES).cpu().numpy()
    assert np.isfinite(Y[:, :64]).all() and np.isnan(Y[:, 64:128]).all() and np.isfinite(Y[:, 128:]).all()
