"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid calls on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from mixed_precision_int_amd import binding as B
from oracle import aq_oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "aq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(aqlib):
    names = declared_functions()
    assert len(names) >= 11
    missing = [n for n in names if not hasattr(aqlib, n)]
    assert not missing, missing
    assert sorted(B.EXPORTS) == names


def test_abi_version_and_status_strings(aqlib):
    assert B.aq_abi_version() == 11
    for code in list(B.STATUS) + [-99]:
        assert aqlib.aq_status_string(code)


def test_act_group_shape_matches_oracle(aqlib):
    # App. B.3: b_M = 1 for one token, 16 otherwise; ceil(M / b_M) x K/64 scales
    for M, K in [(1, 64), (1, 3072), (2, 128), (15, 64), (16, 64), (17, 640), (2048, 2560), (0, 64)]:
        bM, rows, cols = B.aq_act_group_shape(M, K)
        assert bM == O.act_group_rows(M)
        assert (rows, cols) == (-(-M // bM), K // O.ACT_GROUP_K)
        if M:
            _, sxg = O.quant_act_grouped(np.zeros((M, K)))
            assert sxg.shape == (rows, cols)
    for M, K in [(-1, 64), (4, 0), (4, 96)]:
        with pytest.raises(B.AqError) as e:
            B.aq_act_group_shape(M, K)
        assert e.value.status == -2
    x = ctypes.c_int()
    assert aqlib.aq_act_group_shape(4, 64, None, ctypes.byref(x), ctypes.byref(x)) == -1


def test_labels_match_oracle(aqlib):
    rng = np.random.default_rng(0)
    for R, C in [(1, 1), (3, 5), (4, 4), (7, 13), (96, 20)]:
        z = rng.choice([4, 8], size=(R, C))
        assert np.array_equal(B.aq_labels_from_map(z), O.labels_from_map(z))
    with pytest.raises(B.AqError) as e:
        B.aq_labels_from_map(np.array([[4, 5]]))
    assert e.value.status == -4


def test_plan_sizes_match_oracle_pack(aqlib):
    rng = np.random.default_rng(1)
    for N, K, bN, bK in [(256, 512, 64, 128), (192, 640, 64, 64), (6, 96, 3, 32)]:
        z = rng.choice([4, 8], size=(N // bN, K // bK))
        lab = O.labels_from_map(z)
        p = B.aq_plan_pack(N, K, bN, bK, lab)
        pk = O.pack(np.zeros((N, K), np.int64), np.zeros((N, K // bK), np.float32), z, bN, bK)
        assert (p.T4, p.T8) == (pk["T4"], pk["T8"])
        assert p.w4_bytes == pk["w4"].size and p.w8_bytes == pk["w8"].size
        assert p.s4_bytes == 4 * pk["s4"].size and p.s8_bytes == 4 * pk["s8"].size
        assert p.labels_bytes == lab.size and p.offs_bytes == 4 * pk["row_off4"].size
        # eq. 18 with per-row scales, term by term
        total = p.labels_bytes + 2 * p.offs_bytes + p.w4_bytes + p.w8_bytes + p.s4_bytes + p.s8_bytes
        assert total == O.packed_bytes_rowscale(p.T4, p.T8, p.R, p.C, bN, bK)
    with pytest.raises(B.AqError):
        B.aq_plan_pack(256, 512, 64, 48, np.zeros(2, np.uint8))       # bK not a multiple of 32
    with pytest.raises(B.AqError):
        B.aq_plan_pack(250, 512, 64, 128, np.zeros(2, np.uint8))      # N % bN


FAKE = 1 << 20   # 16-byte-aligned fake device address; never dereferenced


def fake_packed(N=256, K=512, bK=128, T4=8, T8=8, **over):
    d = B.AqPacked(N, K, 64, bK, T4, T8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def decode(d, qx=FAKE, sx=FAKE, M=4, bias=None, Y=FAKE, split=1, ws=None, ws_bytes=0):
    return B.lib().aq_linear_decode(ctypes.byref(d), qx, sx, M, bias, Y, split, ws, ws_bytes, None)


def prefill(d, qx=FAKE, sx=FAKE, M=4, bias=None, Y=FAKE, ws=None, ws_bytes=0):
    return B.lib().aq_linear_prefill(ctypes.byref(d), qx, sx, M, bias, Y, ws, ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(bN=32), -3), (dict(bK=96), -3), (dict(N=250), -2),
    (dict(T4=9), -4), (dict(T8=-1), -4), (dict(labels=None), -1), (dict(w8=None), -1),
    (dict(s4=None), -1), (dict(w8=FAKE + 8), -5), (dict(s4=FAKE + 4), -5),
])
def test_packed_descriptor_rejected(aqlib, over, code):
    d = fake_packed(**over)
    assert decode(d) == code
    assert prefill(d) == code


def test_io_rejected(aqlib):
    d = fake_packed()
    assert decode(d, M=-1) == -2
    assert decode(d, M=0) == 0 and prefill(d, M=0) == 0        # no-op, nothing launched
    assert decode(d, qx=None) == -1 and prefill(d, Y=None) == -1
    assert decode(d, qx=FAKE + 1) == -5 and prefill(d, Y=FAKE + 4) == -5
    assert decode(d, bias=FAKE + 4) == -5
    assert decode(d, split=5) == -8                              # not one of 16, 8, 4
    assert decode(d, split=3) == -8
    for sp in (0, 4, 8, 16):
        assert B.lib().aq_workspace_bytes(ctypes.byref(d), 4, 0, sp) == 0
    assert B.lib().aq_workspace_bytes(ctypes.byref(d), 4, 1, 0) == 0   # prefill needs none
    d.labels = FAKE + 2
    assert decode(d) == -5                                       # labels read as 32-bit words


def test_long_prefill_workspace(aqlib):
    """A long prompt on a projection with INT4 tiles needs the temporary INT8
    operand (App. E.3): N*K bytes rounded up to 256, then 4*N*C bytes of
    scales; a missing, short or misaligned workspace is rejected on the host."""
    ws = B.lib().aq_workspace_bytes
    for N, K, bK in [(256, 512, 128), (19456, 2560, 128), (192, 640, 64)]:
        R, C = N // 64, K // bK
        d = fake_packed(N=N, K=K, bK=bK, T4=R * C - 1, T8=1)
        need = ((N * K + 255) // 256) * 256 + 4 * N * C
        assert ws(ctypes.byref(d), 1024, 1, 0) == need
        assert ws(ctypes.byref(d), 8192, 1, 0) == need
        assert ws(ctypes.byref(d), 1023, 1, 0) == 0          # short prompt: on-chip widening
        d8 = fake_packed(N=N, K=K, bK=bK, T4=0, T8=R * C)
        assert ws(ctypes.byref(d8), 4096, 1, 0) == 0         # W8 already in logical order
        assert prefill(d, M=1024) == -6
        assert prefill(d, M=1024, ws=FAKE, ws_bytes=need - 1) == -6
        assert prefill(d, M=1024, ws=FAKE + 4, ws_bytes=need) == -5
        assert B.lib().aq_linear_tile_partials(ctypes.byref(d), FAKE, 1024, 1, FAKE, None, 0, None) == -6
    # beyond 32-bit operand offsets the long route is not taken
    d = fake_packed(N=64, K=1 << 20, bK=128, T4=(1 << 13) - 1, T8=1)
    assert ws(ctypes.byref(d), 4096, 1, 0) == 0


def test_decode_chunk_workspace(aqlib):
    """Decode cuts the input columns into workgroup chunks when the tokens'
    activations for all K would not fit on chip; such a call needs a
    workspace (arrival counters, then FP32 chunk sums) and is rejected on the
    host without one."""
    ws = B.lib().aq_workspace_bytes
    big = fake_packed(N=256, K=65536, T4=4 * 512 - 3, T8=3)
    for M in (5, 16, 33, 64, 100):
        need = ws(ctypes.byref(big), M, 0, 0)
        # the counters sit in a fixed 256 KiB head, then the FP32 chunk sums
        assert need > 256 * 1024 and need % 16 == 0, (M, need)
        assert decode(big, M=M, split=0) == -6
        assert decode(big, M=M, split=0, ws=FAKE, ws_bytes=need - 1) == -6
        assert decode(big, M=M, split=0, ws=FAKE + 4, ws_bytes=need) == -5
        for sp in (16, 8, 4):
            assert ws(ctypes.byref(big), M, 0, sp) > 0
    # one token, or few tokens: per-wave activation slices, no chunks
    for M in (1, 4):
        assert ws(ctypes.byref(big), M, 0, 0) == 0
    # activations fit and the grid already fills the device: no chunks
    wide = fake_packed(N=19456, K=2560, T4=304 * 20 - 7, T8=7)
    assert ws(ctypes.byref(wide), 16, 0, 0) == 0


def test_quant_act_and_partials_rejected(aqlib):
    L = B.lib()
    assert L.aq_quant_act(FAKE, 4, 100, FAKE, FAKE, None) == -2     # K % 64
    assert L.aq_quant_act(FAKE, -1, 128, FAKE, FAKE, None) == -2
    assert L.aq_quant_act(FAKE, 0, 128, FAKE, FAKE, None) == 0
    assert L.aq_quant_act(None, 4, 128, FAKE, FAKE, None) == -1
    assert L.aq_quant_act(FAKE + 4, 4, 128, FAKE, FAKE, None) == -5
    d = fake_packed()
    assert L.aq_linear_tile_partials(ctypes.byref(d), FAKE, 4, 2, FAKE, None, 0, None) == -8
    assert L.aq_linear_tile_partials(ctypes.byref(d), None, 4, 0, FAKE, None, 0, None) == -1
    assert L.aq_linear_tile_partials(ctypes.byref(d), FAKE, 0, 1, FAKE, None, 0, None) == 0


def test_grouped_entry_points_rejected(aqlib):
    """The App. B.3 grouped route validates like the per-token one."""
    L = B.lib()
    assert L.aq_quant_act_grouped(FAKE, 4, 100, FAKE, FAKE, None) == -2      # K % 64
    assert L.aq_quant_act_grouped(FAKE, 0, 128, FAKE, FAKE, None) == 0
    assert L.aq_quant_act_grouped(None, 4, 128, FAKE, FAKE, None) == -1
    assert L.aq_quant_act_grouped(FAKE, 4, 128, FAKE + 4, FAKE, None) == -5
    assert L.aq_quant_act_grouped(FAKE, 16 * 65536, 128, FAKE, FAKE, None) == -2  # row groups > 65535
    d = fake_packed()
    dg = lambda **k: L.aq_linear_decode_grouped(ctypes.byref(d), k.get("qx", FAKE), FAKE, k.get("M", 4), None,
                                                FAKE, k.get("split", 0), None, 0, None)
    assert dg(M=0) == 0 and dg(qx=None) == -1 and dg(qx=FAKE + 1) == -5
    assert dg(split=3) == -8
    assert L.aq_linear_prefill_grouped(ctypes.byref(d), FAKE, None, 4, None, FAKE, None, 0, None) == -1
    assert L.aq_linear_tile_partials_grouped(ctypes.byref(d), FAKE, 0, FAKE, None, 0, None) == 0
    assert L.aq_linear_tile_partials_grouped(ctypes.byref(d), None, 4, FAKE, None, 0, None) == -1
    big = fake_packed(N=256, K=65536, T4=4 * 512 - 3, T8=3)
    assert L.aq_linear_decode_grouped(ctypes.byref(big), FAKE, FAKE, 64, None, FAKE, 0, None, 0, None) == -6


def test_pack_rejects_label_mismatch(aqlib):
    lab = O.labels_from_map(np.full((4, 4), 4))                    # 16 INT4 tiles
    d = fake_packed(T4=8, T8=8)
    assert B.lib().aq_pack_weights(FAKE, lab.ctypes.data, ctypes.byref(d), None) == -4
    assert B.lib().aq_pack_weights(FAKE + 4, lab.ctypes.data, ctypes.byref(d), None) == -5


def test_adaptive_split_bounds(aqlib):
    for N, K in [(256, 512), (5120, 3072), (16384, 3072), (3072, 8192), (2560, 9728)]:
        R, C = N // 64, K // 128
        d = fake_packed(N=N, K=K, T4=R * C, T8=0)
        S = B.lib().aq_decode_split(ctypes.byref(d), 1)
        assert S in (4, 8, 16)


def test_transform_entry_points_rejected(aqlib):
    """App. B.1 transforms: shapes, pointers, alignment and the signed
    permutation tables are checked on the host before any launch."""
    from workloads import gen
    L = B.lib()
    perm, dl, dr = gen.transform_tables()
    t = B.transform_tables(perm, dl, dr)
    T = ctypes.byref(t)
    assert L.aq_transform_rows(FAKE, 4, 100, FAKE, T, FAKE, None) == -2          # K % 64
    assert L.aq_transform_rows(FAKE, 0, 128, FAKE, T, FAKE, None) == 0
    assert L.aq_transform_rows(FAKE, 4, 128, None, T, FAKE, None) == -1
    assert L.aq_transform_rows(FAKE, 4, 128, FAKE, None, FAKE, None) == -1
    assert L.aq_transform_rows(FAKE + 4, 4, 128, FAKE, T, FAKE, None) == -5
    assert L.aq_transform_out(FAKE, -1, 128, FAKE, T, None, FAKE, None) == -2
    assert L.aq_transform_out(FAKE, 4, 128, FAKE, T, FAKE + 4, FAKE, None) == -5   # bias alignment
    q = lambda **k: L.aq_quant_act_transformed(k.get("X", FAKE), k.get("M", 4), k.get("K", 128), k.get("s", FAKE),
                                               k.get("T", T), FAKE, FAKE, None)
    assert q(K=40768 + 64) == -2 and q(K=96) == -2 and q(M=0) == 0
    assert q(s=None) == -1 and q(T=None) == -1 and q(X=FAKE + 4) == -5
    assert L.aq_transform_weights(FAKE, 100, 128, FAKE, FAKE, T, FAKE + (1 << 20), None) == -2
    assert L.aq_transform_weights(FAKE, 64, 128, FAKE, FAKE, T, FAKE + 64 * 128, None) == -8  # overlap
    assert L.aq_transform_weights(FAKE, 64, 128, None, FAKE, T, FAKE + (1 << 20), None) == -1
    bad = perm.copy()
    bad[3, 5] = bad[3, 6]                      # not a permutation
    assert L.aq_transform_rows(FAKE, 4, 128, FAKE, ctypes.byref(B.transform_tables(bad, dl, dr)),
                               FAKE, None) == -8
    bad = perm.copy()
    bad[0, 0] = 64
    assert L.aq_transform_rows(FAKE, 4, 128, FAKE, ctypes.byref(B.transform_tables(bad, dl, dr)),
                               FAKE, None) == -8
    bads = dr.copy()
    bads[5, 63] = 0                            # a sign must be +-1
    assert L.aq_transform_out(FAKE, 4, 128, FAKE, ctypes.byref(B.transform_tables(perm, dl, bads)),
                              None, FAKE, None) == -8


def test_prepared_prefill_rejected(aqlib):
    """The split long-prompt route validates on the host: the preparation
    needs the temporary-operand workspace when the projection has INT4
    tiles (and is a no-op without them); the prepared GEMM needs it for a
    long prompt and not for a short one."""
    L = B.lib()
    d = fake_packed(N=256, K=512, T4=8, T8=8)
    need = L.aq_workspace_bytes(ctypes.byref(d), 1024, 1, 0)
    assert need == 256 * 512 + 4 * 256 * 4
    assert L.aq_prefill_prepare(ctypes.byref(d), None, 0, None) == -6
    assert L.aq_prefill_prepare(ctypes.byref(d), FAKE, need - 1, None) == -6
    assert L.aq_prefill_prepare(ctypes.byref(d), FAKE + 4, need, None) == -5
    d8 = fake_packed(N=256, K=512, T4=0, T8=16)
    assert L.aq_prefill_prepare(ctypes.byref(d8), None, 0, None) == 0          # nothing to prepare
    pp = lambda dd, M, ws=None, n=0: L.aq_linear_prefill_prepared(ctypes.byref(dd), FAKE, FAKE, M, None, FAKE,
                                                                  ws, n, None)
    assert pp(d, 1024) == -6 and pp(d, 1024, FAKE, need - 1) == -6 and pp(d, 1024, FAKE + 4, need) == -5
    assert pp(d, 0) == 0
    assert L.aq_linear_prefill_prepared(ctypes.byref(d), None, FAKE, 4, None, FAKE, None, 0, None) == -1
    assert L.aq_prefill_prepare(ctypes.byref(fake_packed(bK=96)), FAKE, need, None) == -3


def test_prefill_transformed_rejected(aqlib):
    from workloads import gen
    L = B.lib()
    t = B.transform_tables(*gen.transform_tables())
    d = fake_packed()
    f = lambda **k: L.aq_linear_prefill_transformed(ctypes.byref(d), FAKE, FAKE, k.get("M", 4), None,
                                                    k.get("us", FAKE), k.get("t", ctypes.byref(t)), FAKE,
                                                    k.get("ws", None), k.get("n", 0), None)
    assert f(M=0) == 0 and f(us=None) == -1 and f(t=None) == -1
    assert f(M=1024) == -6                     # long prompt with INT4 tiles: the operand workspace


def test_decode_transformed_workspace(aqlib):
    """The transformed decode needs the whole 64-row tile row in one
    workgroup.  Where the plan gives a tile row's row groups to several
    workgroups (few tile rows of many columns) or cuts its columns into
    chunks, the sums meet in a workspace (counters in the fixed 256 KiB
    head, then the sums); where one workgroup holds the tile row (many tile
    rows, or rows short enough for one batch of loads per wave), none is
    needed.  A call without it is rejected on the host."""
    from workloads import gen
    L = B.lib()
    ws = L.aq_workspace_bytes
    t = B.transform_tables(*gen.transform_tables())
    f = lambda d, M, w=None, n=0, split=0, us=FAKE: L.aq_linear_decode_transformed(
        ctypes.byref(d), FAKE, FAKE, M, None, us, ctypes.byref(t), FAKE, split, w, n, None)
    few = fake_packed(N=3072, K=8192, T4=48 * 64 - 5, T8=5)        # 48 tile rows of 64 columns
    short = fake_packed(N=3072, K=3072, T4=48 * 24 - 5, T8=5)      # 48 tile rows of 24 columns
    many = fake_packed(N=16384, K=3072, T4=256 * 24 - 9, T8=9)     # 256 tile rows
    for M in (1, 4, 16):
        need = ws(ctypes.byref(few), M, B.AQ_PHASE_DECODE_TRANSFORMED, 0)
        assert need > 256 * 1024 and need % 16 == 0, (M, need)
        assert ws(ctypes.byref(few), M, B.AQ_PHASE_DECODE, 0) == 0
        assert f(few, M) == -6 and f(few, M, FAKE, need - 1) == -6 and f(few, M, FAKE + 4, need) == -5
        assert ws(ctypes.byref(many), M, B.AQ_PHASE_DECODE_TRANSFORMED, 0) == 0
        assert ws(ctypes.byref(short), M, B.AQ_PHASE_DECODE_TRANSFORMED, 0) == 0
        # a fixed split of 16 waves per row group spreads the tile row over 4 workgroups
        assert ws(ctypes.byref(short), M, B.AQ_PHASE_DECODE_TRANSFORMED, 16) > 256 * 1024
        # a fixed split of 4 waves per row group keeps the tile row in one workgroup
        assert ws(ctypes.byref(few), M, B.AQ_PHASE_DECODE_TRANSFORMED, 4) == 0
    big = fake_packed(N=256, K=65536, T4=4 * 512 - 3, T8=3)        # column chunks
    assert ws(ctypes.byref(big), 16, B.AQ_PHASE_DECODE_TRANSFORMED, 0) >= ws(ctypes.byref(big), 16, 0, 0) > 0
    assert f(many, 0) == 0 and f(many, 4, us=None) == -1 and f(many, 4, split=5) == -8


def test_decode_fp32_workspace(aqlib):
    """Decode from FP32 activations: up to 4 tokens with M*K <= 8192 run as
    one kernel that needs no workspace; other calls quantize into the
    workspace behind a whole block of arrival counters (256 KiB or the
    decode workspace, whichever is larger), then run the decode linear.
    Invalid calls are rejected on the host."""
    L = B.lib()
    ws = L.aq_workspace_bytes
    f = lambda d, M, X=FAKE, w=None, n=0, split=0: L.aq_linear_decode_fp32(
        ctypes.byref(d), X, M, None, FAKE, split, w, n, None)
    q = fake_packed(N=3072, K=3072, T4=48 * 24 - 5, T8=5)         # K = 3072
    d = fake_packed(N=3072, K=8192, T4=48 * 64 - 5, T8=5)         # K = 8192
    for M in (1, 2):
        assert ws(ctypes.byref(q), M, B.AQ_PHASE_DECODE_FP32, 0) == 0, M
    assert ws(ctypes.byref(q), 3, B.AQ_PHASE_DECODE_FP32, 0) > 0
    assert ws(ctypes.byref(d), 1, B.AQ_PHASE_DECODE_FP32, 0) == 0
    for M in (2, 3, 4, 5, 16, 64):
        need = ws(ctypes.byref(d), M, B.AQ_PHASE_DECODE_FP32, 0)
        head = max(ws(ctypes.byref(d), M, B.AQ_PHASE_DECODE, 0), 256 * 1024)
        rows = (M * 8192 + 255) // 256 * 256
        assert need == (head + 255) // 256 * 256 + rows + (4 * M + 255) // 256 * 256, (M, need)
        assert f(d, M) == -6 and f(d, M, w=FAKE, n=need - 1) == -6 and f(d, M, w=FAKE + 4, n=need) == -5
    assert f(q, 4, X=None) == -1 and f(q, 4, X=FAKE + 4) == -5 and f(q, 4, split=5) == -8
    assert f(q, -1) == -2 and f(q, 0, X=None) == 0
