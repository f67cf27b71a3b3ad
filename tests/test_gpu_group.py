"""GPU parity of input-sharing projections packed as one (App. E.4): an
8B-class attention group (q 4096, k 1024, v 1024 rows over K = 4096) and an
MLP group (gate, up 14336 rows each), checked member by member against the
oracle of each member alone."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from mixed_precision_int_amd.model import pack_group, tile_row_slices
from oracle import aq_oracle as O
from tests.parity import assert_output_close, say
from workloads import gen

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _members(names, Ns, K, seed):
    rng = np.random.default_rng(seed)
    ws, zs = [], []
    for i, N in enumerate(Ns):
        ws.append(gen.device_weights(N, K, seed * 10 + i))
        zs.append(gen.map_uniform(rng, N // 64, K // 128, 0.3))
    return ws, zs


@pytest.mark.parametrize("names,Ns,K", [(("q", "k", "v"), (4096, 1024, 1024), 4096),
                                        (("gate", "up"), (14336, 14336), 4096)])
def test_group_members(names, Ns, K):
    ws, zs = _members(names, Ns, K, seed=len(names))
    grp = pack_group(list(names), ws, zs)
    pw = grp.packed
    assert [m[0] for m in grp.members] == list(names)
    assert grp.members[-1][2] == sum(Ns) == pw.N
    # labels and row offsets are those of the concatenated map (eq. 16 over the group)
    z = np.concatenate(zs, axis=0)
    got = tile_row_slices(pw, [0])
    assert np.array_equal(got["labels"], O.labels_from_map(z))
    assert np.array_equal(got["row_off4"], O.row_offsets(z, 4))
    assert np.array_equal(got["row_off8"], O.row_offsets(z, 8))
    rng = np.random.default_rng(9)
    for M in (1, 16, 1040):
        X = gen.acts_outliers(rng, M, K, 4, 20.0)
        qx, sx = aq.aq_quant_act(torch.from_numpy(X).cuda())     # the shared input, once
        Y = (aq.aq_linear_decode(pw, qx, sx) if M <= 64 else aq.aq_linear_prefill(pw, qx, sx))
        torch.cuda.synchronize()
        outs = grp.slices(Y)
        qx_r, sx_r = O.quant_act(X)
        rows = np.arange(M) if M <= 64 else np.array([0, 255, 256, 1039])
        for (name, n0, n1), w, zm in zip(grp.members, ws, zs):
            # two tile rows of the member, its own packing: the member alone
            tr = np.array([0, zm.shape[0] - 1])
            cols = np.concatenate([np.arange(64 * t, 64 * t + 64) for t in tr])
            codes, sW = O.quant_weights(w[torch.from_numpy(cols).cuda()].cpu().numpy(), zm[tr], 64, 128)
            # the member's packed bytes are its own, at the group's offsets
            mine = tile_row_slices(pw, tr + n0 // 64)
            pk = O.pack(codes, sW, zm[tr], 64, 128)
            for k in ("w4", "w8"):
                assert np.array_equal(mine[k], pk[k]), f"{name}: {k}"
            P = O.tile_partials(qx_r[rows], codes, 128)
            y = O.linear_from_partials(P, sx_r[rows], sW)
            c = O.abs_contrib(P, sx_r[rows], sW)
            Yg = outs[name][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
            assert_output_close(Yg, y, c, f"group {'/'.join(names)}: {name} M={M}")
        say(f"  group {names} M={M}: members checked")
