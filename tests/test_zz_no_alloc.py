"""The allocation-free decode entry point (aq_linear_decode_noalloc), for
callers that cannot allocate device memory: its workspace is the library's
own device array.  Checked through the C ABI against aq_linear_decode with a
caller workspace on two calls in a row, the second smaller, both of which
cut the input columns into workgroup chunks (so the array's counters and
chunk sums are used and must be left ready for the next call); plus a call
that needs no workspace and the size limit."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import Case, assert_output_close, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def _case(N, K, M, seed):
    rng = np.random.default_rng(seed)
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, N // 64, K // 128, 0.3)
    X = gen.acts_outliers(rng, M, K, max(1, K // 100), 30.0)
    return W, z, X


def test_noalloc_matches_workspace_decode():
    N, K = 3072, 8192               # Llama-3.2-3B-shaped down projection
    W, z, X = _case(N, K, 64, 31)
    c = Case(W, z, X, name="noalloc")
    pw = c.gpu_pack()
    bias = to_dev(np.random.default_rng(32).standard_normal(N).astype(np.float32))
    for M in (64, 40):              # two calls in a row, the second smaller
        need = aq.aq_workspace_bytes(pw, M, aq.AQ_PHASE_DECODE)
        assert 0 < need <= aq.AQ_DECODE_SCRATCH_BYTES, need
        say(f"  noalloc decode {N}x{K} M={M}: workspace {need} bytes")
        qx, sx = aq.aq_quant_act(to_dev(X[:M]))
        ref = aq.aq_linear_decode(pw, qx, sx, bias=bias)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        aq.aq_linear_decode_noalloc(pw, qx, sx, out, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"M={M}: outputs differ"
        # and the oracle's bar on a few rows
        rows = np.array([0, M // 2, M - 1])
        r = c.ref(None)
        P = O.tile_partials(r["qx"][rows], r["codes"], 128)
        b = bias.cpu().numpy()
        y = O.linear_from_partials(P, r["sx"][rows], r["sW"], b)
        cc = O.abs_contrib(P, r["sx"][rows], r["sW"]) + np.abs(b.astype(np.float64))[None, :]
        assert_output_close(out.cpu().numpy()[rows], y, cc, f"noalloc M={M}")


def test_noalloc_without_chunks_and_limit():
    N, K = 3072, 3072
    W, z, X = _case(N, K, 16, 33)
    c = Case(W, z, X, name="noalloc-small")
    pw = c.gpu_pack()
    qx, sx = c.gpu_quant()
    assert aq.aq_workspace_bytes(pw, 16, aq.AQ_PHASE_DECODE) == 0
    ref = aq.aq_linear_decode(pw, qx, sx)
    out = torch.empty((16, N), dtype=torch.float32, device="cuda")
    aq.aq_linear_decode_noalloc(pw, qx, sx, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # a call whose workspace exceeds the array is refused before any launch
    Wb, zb, _ = _case(3072, 8192, 1, 34)
    pwb = Case(Wb, zb, np.zeros((1, 8192), np.float32)).gpu_pack()
    M = 1024
    assert aq.aq_workspace_bytes(pwb, M, aq.AQ_PHASE_DECODE) > aq.AQ_DECODE_SCRATCH_BYTES
    qx = torch.zeros((M, 8192), dtype=torch.int8, device="cuda")
    sx = torch.ones(M, dtype=torch.float32, device="cuda")
    outb = torch.empty((M, 3072), dtype=torch.float32, device="cuda")
    with pytest.raises(aq.AqError) as e:
        aq.aq_linear_decode_noalloc(pwb, qx, sx, outb)
    assert e.value.status == -6
