"""GPU checks of the split long-prompt route (App. E.3 Prefill): the
temporary INT8 operand prepared by aq_prefill_prepare, on the same stream or
on another one ordered by an event, then aq_linear_prefill_prepared.  Same
kernels as aq_linear_prefill, so the outputs must agree bit for bit; one
case is also held against the oracle on sampled rows to the bar of
tests/parity.py."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import assert_output_close, say, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def setup_case(N, K, bK, M, kind, seed=0):
    rng = np.random.default_rng(seed + N + K + M)
    W = gen.weights(rng, N, K)
    R, C = N // 64, K // bK
    z = {"mixed": gen.map_uniform(rng, R, C, 0.4), "all_int4": np.full((R, C), 4),
         "all_int8": np.full((R, C), 8)}[kind]
    X = gen.acts_heavy_tail(rng, M, K)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK)
    qx, sx = aq.aq_quant_act(to_dev(X))
    return W, z, X, pw, qx, sx


def ws_for(pw):
    return torch.zeros(max(16, aq.aq_workspace_bytes(pw, 1024, aq.AQ_PHASE_PREFILL)), dtype=torch.uint8,
                       device="cuda")


@pytest.mark.parametrize("N,K,bK,M,kind", [
    (256, 1024, 128, 1030, "mixed"),
    (320, 2560, 128, 2048, "all_int4"),
    (256, 640, 64, 1040, "mixed"),
    (256, 1024, 128, 1536, "all_int8"),   # nothing to prepare: the W8 buffer is the operand
    (256, 1024, 128, 100, "mixed"),       # short prompt: the operand is not read
    (6144, 2560, 128, 2048, "mixed"),     # a Qwen3-4B-shaped projection at full size
])
def test_prepared_equals_unsplit(N, K, bK, M, kind):
    W, z, X, pw, qx, sx = setup_case(N, K, bK, M, kind)
    b = to_dev(np.random.default_rng(1).standard_normal(N).astype(np.float32))
    say(f"  prepared {N}x{K}/bK{bK}/M{M}/{kind}")
    Y0 = aq.aq_linear_prefill(pw, qx, sx, b)
    ws = ws_for(pw)
    aq.aq_prefill_prepare(pw, ws)
    Y1 = aq.aq_linear_prefill_prepared(pw, qx, sx, ws, b)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1), f"{N}x{K}/M{M}/{kind}: prepared route differs"


def test_prepared_on_another_stream():
    """The operand of the next projection prepared on a second stream while
    the current GEMM runs; the GEMM stream waits on an event.  Two
    workspaces alternate, each reused only after the GEMM that read it."""
    cases = [setup_case(N, K, 128, 1024, "mixed", seed=s) for s, (N, K) in
             enumerate([(1024, 2560), (512, 4096), (2048, 2560), (512, 9728)])]
    wss = [torch.zeros(max(aq.aq_workspace_bytes(c[3], 1024, aq.AQ_PHASE_PREFILL) for c in cases),
                       dtype=torch.uint8, device="cuda") for _ in range(2)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in cases]
    freed = [torch.cuda.Event() for _ in cases]
    outs = []
    side.wait_stream(main)
    with torch.cuda.stream(side):
        aq.aq_prefill_prepare(cases[0][3], wss[0])
        ready[0].record()
    for i, (W, z, X, pw, qx, sx) in enumerate(cases):
        if i + 1 < len(cases):
            with torch.cuda.stream(side):
                if i >= 1:
                    side.wait_event(freed[i - 1])       # ws (i+1) % 2 was read by GEMM i-1
                aq.aq_prefill_prepare(cases[i + 1][3], wss[(i + 1) % 2])
                ready[i + 1].record()
        main.wait_event(ready[i])
        outs.append(aq.aq_linear_prefill_prepared(pw, qx, sx, wss[i % 2]))
        freed[i].record()
    torch.cuda.synchronize()
    for i, (W, z, X, pw, qx, sx) in enumerate(cases):
        ref = aq.aq_linear_prefill(pw, qx, sx)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], ref), f"case {i}: pipelined prepared route differs"
    # one case against the oracle on sampled rows
    W, z, X, pw, qx, sx = cases[2]
    rows = np.array([0, 1, 511, 512, 1023])
    codes, sW = O.quant_weights(W, z, 64, 128)
    qx_r, sx_r = O.quant_act(X[rows])
    P = O.tile_partials(qx_r, codes, 128)
    assert_output_close(outs[2].cpu().numpy()[rows], O.linear_from_partials(P, sx_r, sW),
                        O.abs_contrib(P, sx_r, sW), "pipelined 2048x2560/M1024")
