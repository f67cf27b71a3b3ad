"""GPU parity of the decode linear from FP32 activations
(aq_linear_decode_fp32) through the C ABI.  Up to 4 tokens with M*K <= 8192
run as one kernel whose workgroups quantize the tokens themselves (App. B.3
per-token rule, eq. 5 rounding); other calls quantize into the workspace and
then decode.  Either way Y must be, bit for bit, that of aq_quant_act
followed by aq_linear_decode with the same split and bias, at every split;
and it must meet the oracle's bar of tests/parity.py."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import assert_output_close, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu

WV = 16  # waves per decode workgroup


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def assert_bits_equal(got, ref, name):
    bad = np.argwhere(bits(got) != bits(ref))
    assert bad.size == 0, f"{name}: {len(bad)} values differ, first {bad[:4].tolist()}"


def setup(N, K, bK, M, seed, X=None):
    rng = np.random.default_rng(seed)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // bK, 0.25)
    if X is None:
        X = gen.acts_outliers(rng, M, K, max(1, K // 100), 25.0)
    b = rng.standard_normal(N).astype(np.float32)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    return pw, W, z, np.ascontiguousarray(X, np.float32), b


def one_kernel(pw, M):
    return M <= 4 and M * pw.K <= 8192


def check_against_two_calls(pw, X, b, name, splits=(0, WV, WV // 2, WV // 4)):
    Xd, bd = to_dev(X), to_dev(b)
    qx, sx = aq.aq_quant_act(Xd)
    for bias in (bd, None):
        for split in splits:
            say(f"  decode_fp32 {name} M={X.shape[0]} split={split} bias={bias is not None} "
                f"one kernel={one_kernel(pw, X.shape[0])}")
            ref = aq.aq_linear_decode(pw, qx, sx, bias=bias, split=split)
            Y = aq.aq_linear_decode_fp32(pw, Xd, bias=bias, split=split)
            torch.cuda.synchronize()
            assert_bits_equal(Y.cpu().numpy(), ref.cpu().numpy(), f"{name}/M{X.shape[0]}/split{split}")


# (name, N, K, b_K, M): the Llama-3.2-3B-shaped projections on the one-kernel
# route (K = 3072: M <= 2; K = 8192: M = 1), a 64 x 64-tile shape (M = 3,
# K = 640), a ragged one (5 tile rows, 9 columns; M = 4, K = 1152), and
# calls past the one-kernel route (M*K > 8192 with M <= 4; M = 5, 16).
CASES = [("qkv", 5120, 3072, 128, 1), ("qkv", 5120, 3072, 128, 2), ("o", 3072, 3072, 128, 3),
         ("o", 3072, 3072, 128, 4), ("gate_up", 16384, 3072, 128, 2), ("down", 3072, 8192, 128, 1),
         ("down", 3072, 8192, 128, 2), ("small64", 256, 640, 64, 3), ("ragged", 320, 1152, 128, 4),
         ("long", 256, 16384, 128, 1), ("down", 3072, 8192, 128, 4), ("o", 3072, 3072, 128, 5),
         ("gate_up", 16384, 3072, 128, 16)]


@pytest.mark.parametrize("name,N,K,bK,M", CASES)
def test_decode_fp32_bit_exact(name, N, K, bK, M):
    pw, W, z, X, b = setup(N, K, bK, M, N + K + M)
    check_against_two_calls(pw, X, b, f"{name} {N}x{K}")


def tie_rows(K, rng):
    """Rows whose quotients x / s sit on and next to rounding ties: row 0 has
    max|x| = 127 (s = 1 exactly) with values k + 1/2 and k + 1/2 -+ 2^-17
    (one FP32 step at that size); row 1 has values (k + 1/2) s rounded to
    FP32 for an inexact s; row 2 is all zero (s = 1e-12, codes 0); row 3
    mixes tiny values (scale floor) with zeros."""
    X = np.zeros((4, K), np.float32)
    k = rng.integers(-127, 127, K).astype(np.float64)
    off = rng.choice([0.0, 2.0 ** -17, -2.0 ** -17], K)
    X[0] = (k + 0.5 + off).astype(np.float32)
    X[0, 0] = 127.0
    s = 3.1 / 127.0
    X[1] = ((rng.integers(-126, 126, K) + 0.5) * s).astype(np.float32)
    X[1, 1] = 3.1
    X[3, ::7] = 1e-11
    return X


@pytest.mark.parametrize("N,K,bK", [(3072, 2048, 128), (256, 4096, 64)])
def test_decode_fp32_ties(N, K, bK):
    """Quotients at and next to rounding ties take the FP64 rule inside the
    one-kernel route (M*K <= 8192 here, except 4 rows of 4096): Y equals that
    of the separate quantizer, bit for bit, for 1, 2 and 4 of these rows."""
    X = tie_rows(K, np.random.default_rng(K))
    pw, W, z, _, b = setup(N, K, bK, 4, 17, X=X)
    for M in (1, 2, 4):
        check_against_two_calls(pw, X[:M].copy(), b, f"ties {N}x{K}", splits=(0,))


@pytest.mark.parametrize("N,K,bK,M", [(3072, 2048, 128, 4), (256, 640, 64, 1), (256, 32768, 128, 8)])
def test_decode_fp32_against_oracle(N, K, bK, M):
    """End to end against the oracle: its per-token quantizer, tile products
    and eq. 19 epilogue with the bias (one-kernel route at M = 4 and 1; the
    workspace route with column chunks at K = 32768, M = 8)."""
    pw, W, z, X, b = setup(N, K, bK, M, 3 * N + M)
    codes, sW = O.quant_weights(W, z, 64, bK)
    qx_r, sx_r = O.quant_act(X)
    P = O.tile_partials(qx_r, codes, bK)
    y = O.linear_from_partials(P, sx_r, sW, b)
    c = O.abs_contrib(P, sx_r, sW) + np.abs(b.astype(np.float64))[None, :]
    say(f"  decode_fp32 {N}x{K}/bK{bK}/M{M} against the oracle")
    Y = aq.aq_linear_decode_fp32(pw, to_dev(X), bias=to_dev(b))
    torch.cuda.synchronize()
    assert_output_close(Y.cpu().numpy(), y, c, f"decode_fp32 {N}x{K}/M{M}")


def test_decode_fp32_calls_in_a_row():
    """One workspace shared by decode calls that cut their columns into
    chunks (arrival counters) and FP32 decode calls that quantize into it
    behind those counters: each result equals its reference and the
    counters are zero at the end."""
    pw, W, z, X, b = setup(256, 32768, 128, 16, 23)
    Xd = to_dev(X)
    qx, sx = aq.aq_quant_act(Xd)
    need = max(aq.aq_workspace_bytes(pw, M, ph, 0) for M in (1, 8, 16)
               for ph in (aq.AQ_PHASE_DECODE, aq.AQ_PHASE_DECODE_FP32))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for M, fp32 in ((16, False), (8, True), (1, True), (16, True), (8, False), (1, False)):
        say(f"  in a row: M={M} fp32={fp32}")
        ref = aq.aq_linear_decode(pw, qx[:M], sx[:M], bias=to_dev(b))
        if fp32:
            Y = aq.aq_linear_decode_fp32(pw, Xd[:M], bias=to_dev(b), ws=ws)
        else:
            Y = aq.aq_linear_decode(pw, qx[:M], sx[:M], bias=to_dev(b), ws=ws)
        torch.cuda.synchronize()
        assert_bits_equal(Y.cpu().numpy(), ref.cpu().numpy(), f"in a row M={M} fp32={fp32}")
    assert int(ws[:4 * 65536].view(torch.int32).abs().sum()) == 0, "arrival counters left set"
