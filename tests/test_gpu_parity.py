"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  The bar is stated in tests/parity.py."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import Case, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def _ragged(N, K, bK, M, seed, frac8=0.5, outliers=3):
    rng = np.random.default_rng(seed)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // bK, frac8)
    X = gen.acts_outliers(rng, M, K, outliers, 20.0)
    return W, z, X


def test_small_workload_all_stages():
    d = gen.small()
    c = Case(d["W"], d["zmap"], d["X"], d["bN"], d["bK"], name="small")
    c.check_all(splits=(0, 2, 4, 8, 16))


def test_small_workload_with_bias():
    d = gen.small()
    b = np.random.default_rng(7).standard_normal(256).astype(np.float32)
    Case(d["W"], d["zmap"], d["X"], bias=b, name="small+bias").check_all(splits=(0, 4, 16))


@pytest.mark.parametrize("N,K,bK,M", [
    (64, 128, 128, 1),       # one tile, one token
    (192, 4736, 128, 17),    # odd tile-row count, 37 tile columns (> 32), ragged M
    (256, 512, 64, 4),       # the pages' 64 x 64 tiles
    (128, 640, 64, 1),
    (384, 2304, 64, 33),     # 36 tile columns at 64 x 64
    (320, 1024, 128, 65),    # M spans two 64-token decode passes
    (256, 512, 128, 130),    # M spans two 128-token prefill blocks, ragged
    (512, 1536, 128, 200),
    (256, 1536, 128, 3),     # 2..4 tokens: per-wave activation slices with MFMA
    (64, 8448, 64, 2),       # 132 tile columns: labels counted from memory
    (128, 10240, 128, 7),    # 16 tokens x K too large for LDS: column chunks
])
def test_ragged_shapes(N, K, bK, M):
    W, z, X = _ragged(N, K, bK, M, seed=N * 7 + K + M)
    Case(W, z, X, 64, bK, name=f"ragged{N}x{K}/bK{bK}/M{M}").check_all(splits=(0, 2, 4, 8, 16))


@pytest.mark.parametrize("N,K,M", [
    (3072, 8192, 16),   # 64 tile columns over 16 waves: 4 per wave, one batch of per-wave slices
    (5120, 3072, 13),   # 2 row groups per workgroup: staged rows (split 16: one row group, slices)
    (768, 2048, 5),     # 10 KB of token rows: staged rows (split 16 too)
    (1024, 8192, 9),    # 64 columns, 4 per wave; 9 tokens, 72 KB of rows: slices
    (1024, 8448, 9),    # 66 columns: 5 per wave, more than one batch: the block's staged token rows
])
def test_decode_private_slices_up_to_16_tokens(N, K, M):
    """5..16 tokens on per-wave activation slices of 4 tiles (two tokens'
    granules per lane slot) where the workgroup holds one row group, each
    wave's columns are one batch and the rows are at least 64 KB, the block's
    staged token rows otherwise;
    the explicit splits move a shape between the two (split 16: one row group
    per workgroup, split 4: four, each wave C/4 columns)."""
    W, z, X = _ragged(N, K, 128, M, seed=N + 3 * K + M)
    bias = np.random.default_rng(M).standard_normal(N).astype(np.float32)
    Case(W, z, X, 64, 128, bias=bias, name=f"priv{N}x{K}/M{M}").check_all(phases=("decode",),
                                                                          splits=(0, 4, 8, 16))


@pytest.mark.parametrize("kind", ["all_int4", "all_int8", "checker", "zero_rows"])
def test_uniform_and_degenerate_maps(kind):
    rng = np.random.default_rng(11)
    N, K, M = 256, 1024, 9
    W = gen.weights(rng, N, K)
    X = gen.acts_outliers(rng, M, K, 4, 30.0)
    R, C = N // 64, K // 128
    if kind == "all_int4":
        z = np.full((R, C), 4)
    elif kind == "all_int8":
        z = np.full((R, C), 8)
    else:
        z = np.where((np.add.outer(np.arange(R), np.arange(C)) % 2) == 0, 4, 8)
    if kind == "zero_rows":
        W[3, :] = 0.0            # every tile row of output 3 is zero: scale 1e-12
        W[70, 128:256] = 0.0     # one zero row segment inside a tile
        X[2, :] = 0.0            # a zero token: scale 1e-12, codes 0
    Case(W, z, X, name=kind).check_all(splits=(0, 4, 16))


def test_extreme_codes_and_ties():
    """Weights and activations that hit +-q_max exactly and round at .5."""
    N, K, M = 128, 256, 3
    W = np.zeros((N, K), np.float32)
    W[:, ::7] = 7.0
    W[:, 1::7] = -2.5
    W[:, 2::7] = 0.5
    W[:, 3::7] = -7.0
    X = np.zeros((M, K), np.float32)
    X[:, ::5] = 127.0
    X[:, 1::5] = -0.5
    X[:, 2::5] = 2.5
    X[:, 3::5] = -127.0
    z = np.array([[4, 8], [8, 4]])
    Case(W, z, X, name="ties").check_all(splits=(0, 4, 8, 16))


def _tie_rows(M, K, seed):
    """Rows whose codes sit on or next to a rounding tie: even rows have
    max |x| = 127 (scale exactly 1) and values k + 1/2 and 1 or 2 ulps from
    it; odd rows have max |x| = 100 (an inexact scale s) and values
    (k + 1/2) s rounded to FP32, so x / s lands within an ulp or so of a
    tie on either side."""
    rng = np.random.default_rng(seed)
    X = np.zeros((M, K), np.float32)
    k = rng.integers(-126, 126, size=(M, K)).astype(np.float64)
    nudge = rng.integers(-2, 3, size=(M, K))
    s_odd = 100.0 / 127.0
    for r in range(M):
        if r % 2 == 0:
            base = (k[r] + 0.5).astype(np.float32)
            X[r, 0] = 127.0
        else:
            base = ((k[r] + 0.5) * s_odd).astype(np.float32)
            X[r, 0] = 100.0
        v = base.copy()
        for step in (1, 2):
            up, dn = nudge[r] == step, nudge[r] == -step
            for _ in range(step):
                v[up] = np.nextafter(v[up], np.float32(np.inf))
                v[dn] = np.nextafter(v[dn], np.float32(-np.inf))
        v[0] = X[r, 0]
        X[r] = v
    return X


@pytest.mark.parametrize("M,K", [
    (3, 3072),      # 1024-thread rows
    (300, 2560),    # 256-thread rows
    (2, 40960),     # few rows past the 1024-thread variants: two-pass loop
    (256, 81984),   # rows past the 256-thread variants: two-pass loop
])
def test_quant_act_near_ties(M, K):
    """Every quantizer route takes its codes from an FP32 estimate of x / s
    where that decides them and from the FP64 division otherwise; exact
    ties and values one or two ulps from a tie, at an exact and an inexact
    scale, must give the oracle's FP64 codes and scales bit for bit."""
    X = _tie_rows(M, K, seed=M + K)
    qx, sx = aq.aq_quant_act(torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    qr, sr = O.quant_act(X)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sr.astype(np.float32).view(np.uint32))
    bad = np.argwhere(qx.cpu().numpy().astype(np.int64) != qr)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("proj", [p[0] for p in gen.LLAMA3B])
def test_llama3b_decode_linears(proj):
    for M in (1, 4, 16):
        d = gen.llama3b_decode(proj, M)
        Case(d["W"], d["zmap"], d["X"], name=d["name"]).check_all(splits=(0,))


@pytest.mark.parametrize("proj", [p[0] for p in gen.QWEN4B])
def test_qwen4b_prefill_linears_sampled_rows(proj):
    """Full M = 2048 in the benchmarked launch shape, i.e. the long-prompt
    route (the temporary INT8 operand, then the 256 x 128 or the persistent
    256 x 256 GEMM): the INT32 tile products of the whole 2048-row call are
    gathered on the device at 48 sampled token rows (every 128-row block
    boundary region, the last row included) and compared bit-exact with the
    oracle; the outputs of the whole call on the same rows meet the bar.  The
    same rows gathered first (a 48-row call, the short route) are checked
    too."""
    d = gen.qwen4b_prefill(proj, 2048)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 127, 128, 1023, 2047], rng.choice(2048, 43, replace=False)]))
    c = Case(d["W"], d["zmap"], d["X"], name=d["name"])
    ref = c.ref(rows)
    c.check_all(rows=rows, phases=("prefill",))
    qx_d, sx_d = c.qx_d, c.sx_d
    M = qx_d.shape[0]
    assert M >= 1024, "the benchmarked prompt takes the long route"
    rows_d = torch.from_numpy(rows).cuda()
    P = aq.aq_linear_tile_partials(c.pw, qx_d, aq.AQ_PHASE_PREFILL)
    P_rows = P.index_select(0, rows_d).cpu().numpy().astype(np.int64)
    del P
    bad = np.argwhere(P_rows != ref["P_rows"])
    assert bad.size == 0, f"{c.name}: {len(bad)} long-route tile products differ, first {bad[:4].tolist()}"
    say(f"  {c.name}: long-route tile products of the M={M} call bit-exact on {len(rows)} rows")
    Y = aq.aq_linear_prefill(c.pw, qx_d, sx_d)
    torch.cuda.synchronize()
    from tests.parity import assert_output_close
    assert_output_close(Y.cpu().numpy()[rows], ref["y_rows"], ref["c_rows"], c.name + "/full-M")


def test_determinism_bitwise():
    d = gen.llama3b_decode("down", 16)
    c = Case(d["W"], d["zmap"], d["X"], name="determinism")
    pw = c.gpu_pack()
    qx, sx = c.gpu_quant()
    a1 = aq.aq_linear_decode(pw, qx, sx).cpu()
    a2 = aq.aq_linear_decode(pw, qx, sx).cpu()
    p1 = aq.aq_linear_prefill(pw, qx, sx).cpu()
    p2 = aq.aq_linear_prefill(pw, qx, sx).cpu()
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    # the two phases agree to the output tolerance
    say("  decode vs prefill max rel diff",
        float((a1 - p1).abs().max() / p1.abs().max()))
    assert float((a1 - p1).abs().max()) <= 1e-4 * float(p1.abs().max())


def test_repeated_calls_split_independent():
    """Every split count gives the same tile products and outputs within the
    bar; the workspace is reused across calls."""
    d = gen.llama3b_decode("qkv", 4)
    c = Case(d["W"], d["zmap"], d["X"], name="splits")
    c.check_all(splits=(4, 8, 16, 0), phases=("decode",))


@pytest.mark.parametrize("M,K", [
    (1, 64),        # one float4 group per lane on a few lanes, most lanes idle
    (3, 3072),      # 1024-thread rows, 3 groups on some lanes
    (16, 8192),
    (5, 17408),     # 1024-thread rows, 5 groups per lane (the longest register variant used)
    (2, 40960),     # few rows too long for the 1024-thread variants: two-pass loop
    (256, 2560),    # 256-thread rows
    (300, 17408),   # 256-thread rows, 17 groups rounded up to 20
    (256, 81984),   # rows too long for the 256-thread variants: two-pass loop
])
def test_quant_act_variants(M, K):
    """Activation codes and scales bit-exact on every launch variant, with a
    zero row, a row whose maximum is negative and a row of ties."""
    rng = np.random.default_rng(M * 131 + K)
    X = gen.acts_outliers(rng, M, K, max(1, K // 100), 30.0)
    X[0, :] = 0.0
    if M > 1:
        X[1, :] = -np.abs(X[1, :])
    if M > 2:
        X[2, :] = np.resize(np.array([127.0, -0.5, 2.5, -127.0, 1.5], np.float32), K)
    qx_ref, sx_ref = O.quant_act(X)
    qx, sx = aq.aq_quant_act(to_dev(X))
    torch.cuda.synchronize()
    say(f"  quant_act M={M} K={K}")
    assert np.array_equal(qx.cpu().numpy().astype(np.int64), qx_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("N,K,bK,M,kind", [
    (256, 512, 128, 1030, "mixed"),     # 4 tile columns: only the guarded tail of the column loop
    (192, 1536, 128, 1024, "mixed"),    # 3 tile rows (partial N block), 12 columns = 2 unrolled groups
    (320, 2560, 128, 1100, "mixed"),    # 20 columns: 3 groups + a 2-column tail; ragged M
    (128, 128, 128, 1024, "mixed"),     # a single tile column
    (256, 640, 64, 1040, "mixed"),      # 64 x 64 tiles
    (256, 1024, 128, 2048, "all_int4"),
    (256, 1024, 128, 1536, "all_int8"), # W8 already in logical order: no temporary buffer
])
def test_long_prefill_temporary_int8(N, K, bK, M, kind):
    """Prompts of >= 1024 rows: the selected weights are expanded once per
    call to INT8 tiles in logical order and the GEMM runs over them (App. E.3
    Prefill); tile products on every row and outputs against the oracle."""
    rng = np.random.default_rng(N + K + M)
    W = gen.weights(rng, N, K)
    R, C = N // 64, K // bK
    z = {"mixed": gen.map_uniform(rng, R, C, 0.4), "all_int4": np.full((R, C), 4),
         "all_int8": np.full((R, C), 8)}[kind]
    X = gen.acts_heavy_tail(rng, M, K)
    bias = rng.standard_normal(N).astype(np.float32)
    need = aq.aq_workspace_bytes(Case(W, z, X, 64, bK).gpu_pack(), M, aq.AQ_PHASE_PREFILL)
    assert (need == 0) == (kind == "all_int8")
    Case(W, z, X, 64, bK, bias=bias, name=f"long{N}x{K}/bK{bK}/M{M}/{kind}").check_all(phases=("prefill",))


@pytest.mark.parametrize("N,K,bK,M,kind", [
    (256, 8192, 128, 64, "mixed"),      # 64 tokens x 8192 columns: several chunks
    (192, 5120, 128, 37, "mixed"),      # ragged tokens: 3 groups of 16, last partial
    (320, 17408, 128, 33, "mixed"),     # 136 tile columns: labels counted from memory
    (128, 8192, 64, 20, "mixed"),       # 64 x 64 tiles
    (128, 4096, 128, 100, "mixed"),     # two 64-token chunks along the grid's y
    (256, 6144, 128, 48, "all_int4"),
    (256, 6144, 128, 48, "all_int8"),
])
def test_decode_chunked_columns(N, K, bK, M, kind):
    """Decode with the input columns cut into workgroup chunks (staged
    activations of all K would not fit on chip, or the grid would leave CUs
    idle): FP32 chunk sums through the workspace, added in increasing chunk
    order by the row block's last workgroup.  Tile products, outputs for the
    adaptive and every explicit split, and bitwise-repeatable outputs (the
    arrival counters are left at zero by every call)."""
    rng = np.random.default_rng(N + 3 * K + M)
    W = gen.weights(rng, N, K)
    R, C = N // 64, K // bK
    z = {"mixed": gen.map_uniform(rng, R, C, 0.3), "all_int4": np.full((R, C), 4),
         "all_int8": np.full((R, C), 8)}[kind]
    X = gen.acts_outliers(rng, M, K, 5, 25.0)
    bias = rng.standard_normal(N).astype(np.float32)
    c = Case(W, z, X, 64, bK, bias=bias, name=f"chunked{N}x{K}/bK{bK}/M{M}/{kind}")
    Wv = 16  # waves per decode workgroup
    out = c.check_all(phases=("decode",), splits=(0, Wv, Wv // 2, Wv // 4))
    assert aq.aq_workspace_bytes(c.pw, M, aq.AQ_PHASE_DECODE) > 0
    bias_d = to_dev(bias)
    for s in (0, Wv // 4):
        again = aq.aq_linear_decode(c.pw, c.qx_d, c.sx_d, bias_d, split=s)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), out[f"decode{s}"].view(torch.int32)), s


def test_decode_chunked_interleaved_calls():
    """Back-to-back decode calls on one stream and one workspace, cycling
    through projections whose chunk layouts differ (chunk counts, row
    blocks, token groups): every output of every call matches the oracle.
    A chunk sum read before its writer's store is visible device-wide, or an
    arrival counter not left at zero, returns another call's data."""
    shapes = [(6144, 4096, 64), (4096, 14336, 64), (2048, 8192, 40), (1024, 17408, 33)]
    cases = []
    for i, (N, K, M) in enumerate(shapes):
        rng = np.random.default_rng(900 + i)
        W = gen.weights(rng, N, K)
        z = gen.map_uniform(rng, N // 64, K // 128, 0.3)
        X = gen.acts_outliers(rng, M, K, 4, 20.0)
        c = Case(W, z, X, name=f"interleaved{N}x{K}/M{M}")
        ref = c.ref(np.arange(M))
        c.gpu_pack()
        c.gpu_quant()
        assert aq.aq_workspace_bytes(c.pw, M, aq.AQ_PHASE_DECODE) > 0, c.name
        cases.append((c, ref))
    outs = []
    for rep in range(12):
        for c, _ in cases:
            outs.append((c, aq.aq_linear_decode(c.pw, c.qx_d, c.sx_d)))
    torch.cuda.synchronize()
    from tests.parity import assert_output_close
    refs = {id(c): r for c, r in cases}
    for k, (c, Y) in enumerate(outs):
        r = refs[id(c)]
        assert_output_close(Y.cpu().numpy(), r["y_rows"], r["c_rows"], f"{c.name}/call{k}")


def test_decode_chunked_many_token_chunks():
    """More row blocks x token chunks than a decode workspace has arrival
    counters (65536): the call runs as several launches along the token
    axis.  N = 65536 (1024 row blocks), K = 4096, M = 4160 tokens (65 chunks
    of 64); outputs on three tile rows x six tokens that span both launches
    against the oracle."""
    N, K, M = 65536, 4096, 4160
    R, C = N // 64, K // 128
    rng = np.random.default_rng(4242)
    zmap = gen.map_uniform(rng, R, C, 0.3)
    W = gen.device_weights(N, K, 4243)
    pw = aq.aq_pack_weights(W, aq.aq_labels_from_map(zmap.astype(np.uint8)), 64, 128)
    X = gen.device_acts_outliers(M, K, 4244)
    qx, sx = aq.aq_quant_act(X)
    Y = aq.aq_linear_decode(pw, qx, sx)
    torch.cuda.synchronize()
    tile_rows = np.array([0, 333, R - 1])
    cols = np.concatenate([np.arange(64 * r, 64 * r + 64) for r in tile_rows])
    tokens = np.array([0, 63, 64, 4095, 4096, M - 1])
    W_sub = W[torch.from_numpy(cols).cuda()].cpu().numpy()
    X_rows = X[torch.from_numpy(tokens).cuda()].cpu().numpy()
    Y_g = Y[torch.from_numpy(tokens).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    del W, Y
    codes, sW = O.quant_weights(W_sub, zmap[tile_rows], 64, 128)
    qx_ref, sx_ref = O.quant_act(X_rows)
    P = O.tile_partials(qx_ref, codes, 128)
    from tests.parity import assert_output_close
    assert_output_close(Y_g, O.linear_from_partials(P, sx_ref, sW), O.abs_contrib(P, sx_ref, sW),
                        "many-token-chunks")


@pytest.mark.parametrize("N,K,M", [(1024, 4096, 1), (1024, 4096, 4), (1024, 4096, 16), (9536, 2048, 40),
                                   (576, 16384, 3)])
def test_decode_inline_metadata(N, K, M):
    """The host metadata image (one record per tile row: row offsets, then
    the row's labels as 128 bits) matches the oracle's offsets and labels,
    and decode gives bitwise the same outputs whether the image travels in
    the kernel arguments or the metadata is read from device memory."""
    rng = np.random.default_rng(N + K + M)
    R, C = N // 64, K // 128
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, R, C, 0.35)
    X = gen.acts_outliers(rng, M, K, 3, 20.0)
    c = Case(W, z, X, name=f"inline-meta{N}x{K}/M{M}")
    out = c.check_all(phases=("decode",))
    meta = c.pw.meta_host.reshape(R, 6)
    assert np.array_equal(meta[:, 0].astype(np.int64), O.row_offsets(z, 4)[:R])
    assert np.array_equal(meta[:, 1].astype(np.int64), O.row_offsets(z, 8)[:R])
    bits = (np.asarray(z) == 4).astype(np.uint64)
    for r in range(R):
        want = [int(sum(int(bits[r, j]) << (j - 32 * w) for j in range(32 * w, min(C, 32 * w + 32))))
                for w in range(4)]
        assert [int(v) for v in meta[r, 2:]] == want, r
    saved = c.pw.desc.meta_host
    try:
        c.pw.desc.meta_host = None     # device metadata route
        Y = aq.aq_linear_decode(c.pw, c.qx_d, c.sx_d)
        torch.cuda.synchronize()
    finally:
        c.pw.desc.meta_host = saved
    assert torch.equal(Y.view(torch.int32), out["decode0"].view(torch.int32))


def test_long_prefill_persistent_tiles_ragged():
    """The persistent 256 x 256-tile kernel (taken when the prompt yields at
    least one tile per compute unit): 257 tile rows (the last N block holds
    one), 1040 tokens (the last M block holds 16), two tile columns, a bias;
    tile products on every row and outputs against the oracle."""
    N, K, M = 16448, 256, 1040
    rng = np.random.default_rng(77)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // 128, 0.35)
    X = gen.acts_heavy_tail(rng, M, K)
    bias = rng.standard_normal(N).astype(np.float32)
    Case(W, z, X, 64, 128, bias=bias, name="persistent16448x256/M1040").check_all(phases=("prefill",))


@pytest.mark.parametrize("N,K,M", [(256, 8192, 64), (192, 5120, 37), (1024, 14336, 24), (256, 8192, 100)])
def test_short_prefill_on_decode_with_handover(N, K, M):
    """A prompt of at most 64 rows (128 on a projection too narrow for the
    GEMM grid, 256 x 8192 at M = 100) runs on the decode kernels; where their
    plan cuts the columns into chunks, the prefill call's workspace (handed
    in uninitialized: filled with 0xFF here) serves as the decode workspace
    after the call zeroes its counters.  Outputs against the oracle, the same
    bits as the decode call, twice in a row on the same dirty workspace."""
    rng = np.random.default_rng(7 * N + K + M)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // 128, 0.3)
    X = gen.acts_outliers(rng, M, K, 5, 25.0)
    bias = rng.standard_normal(N).astype(np.float32)
    c = Case(W, z, X, 64, 128, bias=bias, name=f"shortprefill{N}x{K}/M{M}")
    c.check_all(phases=("prefill",))
    need = aq.aq_workspace_bytes(c.pw, M, aq.AQ_PHASE_PREFILL)
    assert need >= aq.aq_workspace_bytes(c.pw, M, aq.AQ_PHASE_DECODE) > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    bias_d = to_dev(bias)
    ref = aq.aq_linear_decode(c.pw, c.qx_d, c.sx_d, bias_d)
    for _ in range(2):
        Y = aq.aq_linear_prefill(c.pw, c.qx_d, c.sx_d, bias_d, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), ref.view(torch.int32))
        ws.fill_(0xFF)
