"""GPU parity of the fitted weight scales (App. B.2 eq. 7, aq_pack_weights_mse)
against the oracle: packed bytes and scale bits bit-exact, and the linear
outputs of the packed model within the bar of tests/parity.py."""
import numpy as np
import pytest
import torch

import mixed_precision_int_amd as aq
from oracle import aq_oracle as O
from tests.parity import assert_output_close, assert_packed_equal, packed_to_host, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,bK,kind", [(256, 512, 128, "mixed"), (128, 256, 64, "mixed"),
                                         (192, 384, 128, "all_int4"), (64, 256, 128, "all_int8")])
def test_mse_pack_bit_exact(N, K, bK, kind):
    rng = np.random.default_rng(N + K + bK)
    W = gen.weights(rng, N, K)
    W[0, :bK] = 0.0                                   # a zero segment: the 1e-12 floor
    W[1, :bK] *= 0.0; W[1, 3] = 0.5; W[1, 7] = -0.25  # a sparse segment
    R, C = N // 64, K // bK
    z = {"mixed": gen.map_uniform(rng, R, C, 0.4), "all_int4": np.full((R, C), 4),
         "all_int8": np.full((R, C), 8)}[kind]
    codes, sW = O.quant_weights_mse(W, z, 64, bK)
    pw = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, bK, mse=True)
    assert_packed_equal(packed_to_host(pw), O.pack(codes, sW, z, 64, bK), f"mse{N}x{K}/bK{bK}/{kind}")
    # the linear path reads the fitted scales like any packed projection
    X = gen.acts_outliers(rng, 5, K, 2, 20.0)
    qx_r, sx_r = O.quant_act(X)
    P = O.tile_partials(qx_r, codes, bK)
    qx, sx = aq.aq_quant_act(to_dev(X))
    for Y, tag in ((aq.aq_linear_decode(pw, qx, sx), "decode"), (aq.aq_linear_prefill(pw, qx, sx), "prefill")):
        torch.cuda.synchronize()
        assert_output_close(Y.cpu().numpy(), O.linear_from_partials(P, sx_r, sW), O.abs_contrib(P, sx_r, sW),
                            f"mse{N}x{K}/{tag}")


def test_mse_scales_differ_from_absmax_and_fit_better():
    """On Gaussian weights the fitted scales differ from the absmax ones on
    most rows and never reconstruct worse (eq. 7 includes the endpoint scale)."""
    rng = np.random.default_rng(4)
    N, K = 128, 256
    W = gen.weights(rng, N, K)
    z = gen.map_uniform(rng, 2, 2, 0.5)
    pa = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128)
    pm = aq.aq_pack_weights(to_dev(W), aq.aq_labels_from_map(z.astype(np.uint8)), 64, 128, mse=True)
    def recon(pw):
        codes, sW, _ = O.unpack(packed_to_host_full(pw, z))
        return codes * np.repeat(np.asarray(sW, np.float64), 128, axis=1)
    ea = np.sum((recon(pa) - W) ** 2, axis=1)
    em = np.sum((recon(pm) - W) ** 2, axis=1)
    assert np.all(em <= ea * (1 + 1e-6) + 1e-30)
    assert np.mean(em < ea) > 0.5


def packed_to_host_full(pw, z):
    d = packed_to_host(pw)
    d.update(N=pw.plan.N, K=pw.plan.K, bN=64, bK=pw.plan.bK)
    return d
