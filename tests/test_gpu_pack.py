"""GPU parity of the offline quantise + pack step: the packed bytes, scales and
zero-points written by the HIP kernel are bit-identical to the oracle's, and the
canonical view read back by w4a16_unpack equals the oracle's codes."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _check_packed(o, pw):
    import torch
    torch.cuda.synchronize()
    qw = pw.qweight.cpu().numpy()
    assert np.array_equal(qw, o["qweight"]), f"qweight differs at {np.count_nonzero(qw != o['qweight'])} bytes"
    s = pw.scales.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(s, o["scales_dev"]), "scales differ"
    z = pw.zeros.cpu().numpy().view(np.uint32)
    assert np.array_equal(z, o["zeros_dev"]), "zeros differ"
    codes, s_out, z_out = H.lib().unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), o["codes"])
    assert np.array_equal(s_out.cpu().numpy().view(np.uint16), o["s_bits"])
    assert np.array_equal(z_out.cpu().numpy(), o["zeros"])


@pytest.mark.parametrize("N,K,group", [(8, 32, 32), (72, 64, 32), (200, 96, 32), (136, 256, 64),
                                       (64, 384, 128), (328, 640, 128), (1000, 1024, 64)])
def test_pack_small_shapes_bit_exact(N, K, group):
    w = wl.random_weights(N * 7 + K, N, K, scale=0.05)
    w[0, :group] = 0.0                         # degenerate all-zero group
    w[1 % N, :group] = np.abs(w[1 % N, :group])  # one-signed group
    o = H.oracle_pack(w, group)
    _check_packed(o, H.gpu_pack(w, group))


def test_pack_constructed_ties_and_edges():
    N, K, group = 16, 128, 128
    s = 2.0 ** -6
    j = np.arange(-8, 7)
    row = np.concatenate([[-8 * s, 7 * s], (j + 0.5) * s, np.zeros(K - 2 - j.size)])
    w = np.tile(row.astype(np.float32), (N, 1))
    w[1] = 1e-12                     # scale underflows fp16 -> 2^-24
    w[2] = 0.5                       # constant positive
    w[3] = -0.5                      # constant negative
    w[4] = np.float32(2.0 ** 17)     # near the documented |w| bound
    w[5] = np.float32(-1.5e-39)      # fp32 subnormal weights
    o = H.oracle_pack(w, group)
    _check_packed(o, H.gpu_pack(w, group))


@pytest.mark.slow
@pytest.mark.parametrize("cfg,mat", [(1, 0), (2, 0), (2, 4), (2, 6), (3, 0), (4, 0), (5, 0)])
def test_pack_full_size_configs_bit_exact(cfg, mat):
    group = wl.WORKLOADS[cfg].group
    w, o, pw = H.prepared((cfg, mat), lambda: wl.weights(cfg, mat), group)
    _check_packed(o, pw)
    # the round-trip bound holds on every element of the configuration
    wv = w.reshape(w.shape[0], -1, group)
    s = ref.f16_bits_to_f64(o["s_bits"]).T[:, :, None]
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group).reshape(wv.shape)
    inner = (o["codes"].reshape(wv.shape) > 0) & (o["codes"].reshape(wv.shape) < 15)
    err = np.abs(wv.astype(np.float64) - w_hat)
    assert np.all(err[inner] <= (0.5 * s + 2.0 ** -24 * np.abs(wv))[inner])
