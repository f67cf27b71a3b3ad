"""GPU parity of the pages' activation quantizer (App. B.3: 64-feature x b_M-row
groups, eq. 6 endpoint scale) and of the grouped eq. 19, through the C ABI,
against the oracle.  Bar as in tests/parity.py: codes, scale bits and INT32
group products bit-exact; outputs within 1e-4 normwise and componentwise."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import assert_output_close, assert_packed_equal, packed_to_host, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def run_case(N, K, bK, M, kind="mixed", bias=False, seed=0, splits=(0,), phases=("decode", "prefill")):
    rng = np.random.default_rng(seed + N + 3 * K + 7 * M)
    W = gen.weights(rng, N, K)
    R, C = N // 64, K // bK
    z = {"mixed": gen.map_uniform(rng, R, C, 0.35), "all_int4": np.full((R, C), 4),
         "all_int8": np.full((R, C), 8)}[kind]
    X = gen.acts_outliers(rng, M, K, 4, 25.0)
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    name = f"grouped{N}x{K}/bK{bK}/M{M}/{kind}{'+bias' if bias else ''}"
    say(f"[{name}]")
    # oracle
    codes, sW = O.quant_weights(W, z, 64, bK)
    qx_r, sxg_r = O.quant_act_grouped(X)
    P_r = O.group_partials(qx_r, codes)
    y_r = O.linear_from_group_partials(P_r, sxg_r, sW, bK, b)
    c_r = O.abs_contrib_grouped(P_r, sxg_r, sW, bK)
    if b is not None:
        c_r = c_r + np.abs(b.astype(np.float64))[None, :]
    # HIP path
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    assert_packed_equal(packed_to_host(pw), O.pack(codes, sW, z, 64, bK), name)
    qx, sxg = aq.aq_quant_act_grouped(to_dev(X))
    torch.cuda.synchronize()
    assert np.array_equal(qx.cpu().numpy().astype(np.int64), qx_r), f"{name}: codes differ"
    assert np.array_equal(sxg.cpu().numpy().view(np.uint32), sxg_r.view(np.uint32)), f"{name}: scale bits differ"
    P = aq.aq_linear_tile_partials_grouped(pw, qx)
    torch.cuda.synchronize()
    bad = np.argwhere(P.cpu().numpy().astype(np.int64) != P_r)
    assert bad.size == 0, f"{name}: {len(bad)} group products differ, first {bad[:4].tolist()}"
    bd = None if b is None else to_dev(b)
    outs = {}
    if "decode" in phases:
        for s in splits:
            Y = aq.aq_linear_decode_grouped(pw, qx, sxg, bd, split=s)
            torch.cuda.synchronize()
            assert_output_close(Y.cpu().numpy(), y_r, c_r, f"{name}/decode/split{s}")
            outs[f"decode{s}"] = Y
    if "prefill" in phases:
        Y = aq.aq_linear_prefill_grouped(pw, qx, sxg, bd)
        torch.cuda.synchronize()
        assert_output_close(Y.cpu().numpy(), y_r, c_r, f"{name}/prefill")
        outs["prefill"] = Y
    return outs


@pytest.mark.parametrize("M", [1, 2, 4, 5, 15, 16, 17, 33, 64, 100])
def test_grouped_token_counts(M):
    """b_M = 1 for one token (the vector-ALU path), 16 otherwise, with
    ragged last groups; every decode split the kernel offers."""
    Wv = 16  # waves per decode workgroup
    run_case(256, 1024, 128, M, splits=(0, Wv, Wv // 2, Wv // 4), bias=(M % 2 == 1))


@pytest.mark.parametrize("kind", ["all_int4", "all_int8"])
@pytest.mark.parametrize("M", [1, 24])
def test_grouped_uniform_maps(kind, M):
    run_case(192, 768, 128, M, kind=kind)


@pytest.mark.parametrize("M", [1, 3, 20])
def test_grouped_tile64(M):
    """64 x 64 tiles: one activation group per tile."""
    run_case(256, 512, 64, M, bias=True)


def test_grouped_chunked_columns():
    """Large M*K: column chunks through the workspace, grouped scales."""
    N, K, M = 256, 8192, 64
    pw_need = run_case(N, K, 128, M, phases=("decode",))
    assert "decode0" in pw_need


def test_grouped_long_prompt():
    """A prompt of 1040 rows (65 groups of 16, the last one ragged) on the
    any-length route; also the 32-token-group plan of projections larger
    than 16 MB is exercised by the model-size case below."""
    run_case(512, 1024, 128, 1040, phases=("prefill",), bias=True)


def test_grouped_large_projection_sampled():
    """A 19456 x 2560 projection (> 16 MB packed: 32-token groups) at M = 48;
    outputs of every token on three tile rows against the oracle."""
    N, K, M = 19456, 2560, 48
    R, C = N // 64, K // 128
    rng = np.random.default_rng(31)
    z = gen.map_uniform(rng, R, C, 0.3)
    Wd = gen.device_weights(N, K, 77)
    pw = aq.aq_pack_weights(Wd, aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
    X = gen.acts_outliers(rng, M, K, 4, 25.0)
    qx, sxg = aq.aq_quant_act_grouped(to_dev(X))
    Y = aq.aq_linear_decode_grouped(pw, qx, sxg)
    torch.cuda.synchronize()
    tile_rows = np.array([0, 151, R - 1])
    cols = np.concatenate([np.arange(64 * r, 64 * r + 64) for r in tile_rows])
    codes, sW = O.quant_weights(Wd[torch.from_numpy(cols).cuda()].cpu().numpy(), z[tile_rows], 64, 128)
    qx_r, sxg_r = O.quant_act_grouped(X)
    P_r = O.group_partials(qx_r, codes)
    assert_output_close(Y[:, torch.from_numpy(cols).cuda()].cpu().numpy(),
                        O.linear_from_group_partials(P_r, sxg_r, sW, 128),
                        O.abs_contrib_grouped(P_r, sxg_r, sW, 128), "grouped-19456x2560/M48")


@pytest.mark.parametrize("N,K,M,kind", [(192, 1536, 1030, "mixed"),    # a partial N block, ragged M
                                        (256, 1024, 2048, "all_int4"),
                                        (320, 2560, 1024, "all_int8")])  # W8 in place: no operand
def test_grouped_long_route(N, K, M, kind):
    """Long prompts take the long-prompt GEMM with the two 64-feature halves
    of every tile kept apart (App. B.3 groups in eq. 19): group products of
    every row bit-exact, outputs within the bar, with a bias."""
    run_case(N, K, 128, M, kind=kind, bias=True, phases=("prefill",))


def test_grouped_long_route_full_size_sampled():
    """Qwen3-4B-shaped qkv (6144 x 2560) at M = 2048 on the long route: the
    INT32 group products of the whole call gathered on the device at sampled
    token rows (every 16-row group boundary region, each of a block's four
    64-row waves) bit-exact, and the outputs of the whole call on those rows
    within the bar."""
    d = gen.qwen4b_prefill("qkv", 2048)
    W, z, X = d["W"], d["zmap"], d["X"]
    M = X.shape[0]
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 15, 16, 63, 64, 127, 128, 191, 255, 1024, M - 1],
                                     rng.choice(M, 9, replace=False)]))
    codes, sW = O.quant_weights(W, z, 64, 128)
    qx_r, sxg_r = O.quant_act_grouped(X)
    P_r = O.group_partials(qx_r[rows], codes)
    # the grouped eq. 19 on the sampled rows: scales of each row's 16-row group
    sxr = sxg_r[rows // 16]
    y_r = np.zeros((len(rows), W.shape[0]))
    c_r = np.zeros_like(y_r)
    for c in range(K_GROUPS(X)):
        t = (sxr[:, c].astype(np.float64)[:, None] * sW[None, :, c // 2].astype(np.float64)) * P_r[:, :, c]
        y_r += t
        c_r += np.abs(t)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
    qx, sxg = aq.aq_quant_act_grouped(to_dev(X))
    assert aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL_GROUPED) == aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL)
    rows_d = torch.from_numpy(rows).cuda()
    P = aq.aq_linear_tile_partials_grouped(pw, qx)
    P_g = P.index_select(0, rows_d).cpu().numpy().astype(np.int64)
    del P
    bad = np.argwhere(P_g != P_r)
    assert bad.size == 0, f"grouped qkv/M2048: {len(bad)} group products differ, first {bad[:4].tolist()}"
    Y = aq.aq_linear_prefill_grouped(pw, qx, sxg)
    torch.cuda.synchronize()
    assert_output_close(Y.index_select(0, rows_d).cpu().numpy(), y_r, c_r, "grouped qkv/M2048 (long route)")


def K_GROUPS(X):
    return X.shape[1] // 64


def test_grouped_long_route_after_nan_in_lds():
    """The grouped long-prompt GEMM reads no LDS it has not written: run
    right after a kernel that leaves NaN across every compute unit's LDS (the
    one-pass transformed quantizer staging 512 rows of 40768 features with an
    invalid seed, 160 KiB of NaN per row), its outputs stay finite and within
    the bar.  Column 0 has no previous column whose second-group scales it
    would rescale; reading that unloaded stage slot once turned rows NaN."""
    N, K, M = 512, 1024, 1040
    rng = np.random.default_rng(1234)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // 128, 0.35)
    X = gen.acts_outliers(rng, M, K, 4, 25.0)
    b = rng.standard_normal(N).astype(np.float32)
    codes, sW = O.quant_weights(W, z, 64, 128)
    qx_r, sxg_r = O.quant_act_grouped(X)
    P_r = O.group_partials(qx_r, codes)
    y_r = O.linear_from_group_partials(P_r, sxg_r, sW, 128, b)
    c_r = O.abs_contrib_grouped(P_r, sxg_r, sW, 128) + np.abs(b.astype(np.float64))[None, :]
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
    qx, sxg = aq.aq_quant_act_grouped(to_dev(X))
    bd = to_dev(b)
    ws = torch.empty(max(16, aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_PREFILL_GROUPED)), dtype=torch.uint8,
                     device="cuda")
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Kn = 40768
    Xn = torch.ones((512, Kn), dtype=torch.float32, device="cuda")
    qn, sn = aq.aq_quant_act_transformed(Xn, np.full(Kn // 64, 9, np.int8), gen.transform_tables())
    torch.cuda.synchronize()
    assert torch.isnan(sn).all(), "the planting kernel did not stage NaN"
    say(f"  grouped long route {N}x{K}/M{M} right after NaN in LDS")
    aq.aq_linear_prefill_grouped(pw, qx, sxg, bd, out=Y, ws=ws)
    torch.cuda.synchronize()
    assert_output_close(Y.cpu().numpy(), y_r, c_r, "grouped long route after NaN in LDS")
