"""GPU parity of the grouped call (w4a16_linear_group): several layers of one
M, K, group and type in one launch give, for every problem, the bits of
w4a16_linear on that problem alone, and stay within the oracle's bar."""
import numpy as np
import pytest

import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu

K, GROUP = 1024, 64
NS = (1000, 520, 136)


def _weights(N):
    return H.prepared(("group", N, K, GROUP), lambda: wl.random_weights(3 * N + K, N, K), GROUP)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 3, 16, 40, 300])
@pytest.mark.parametrize("shared_x", [False, True])
def test_group_matches_single_calls(dtype, M, shared_x):
    import torch
    probs = [_weights(N) for N in NS]
    xbits = [wl.random_activations(11 * M + p, M, K, dtype) for p in range(len(NS))]
    if shared_x:
        xbits = [xbits[0]] * len(NS)
    xs = [H.to_device_bits(b, dtype) for b in xbits]
    if shared_x:
        xs = [xs[0]] * len(NS)
    ys = H.lib().linear_group(xs, [pw for _, _, pw in probs])
    torch.cuda.synchronize()
    for p, (w, o, pw) in enumerate(probs):
        single = H.lib().linear(xs[p], pw)
        torch.cuda.synchronize()
        assert ys[p].shape == (M, NS[p])
        assert torch.equal(ys[p].view(torch.int16), single.view(torch.int16)), p
        H.check_against_oracle(ys[p], xbits[p], dtype, o, GROUP)


def test_group_of_one_and_of_eight():
    import torch
    w, o, pw = _weights(1000)
    xb = wl.random_activations(5, 2, K, "f16")
    x = H.to_device_bits(xb, "f16")
    (y1,) = H.lib().linear_group([x], [pw])
    y8 = H.lib().linear_group([x] * 8, [pw] * 8)
    torch.cuda.synchronize()
    for y in y8:
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    H.check_against_oracle(y1, xb, "f16", o, 64)


@pytest.mark.slow
def test_group_decode_layer_set_full_size():
    """q, k, v of the 13B decode layer set in one launch, then gate and up."""
    import torch
    cfg = 2
    wlc = wl.WORKLOADS[cfg]
    for mats in ((0, 1, 2), (4, 5)):
        probs = [H.prepared((cfg, m), lambda m=m: wl.weights(cfg, m), wlc.group) for m in mats]
        xbits = [wl.activations(cfg, m, 1) for m in mats]
        xs = [H.to_device_bits(b, wlc.dtype) for b in xbits]
        ys = H.lib().linear_group(xs, [pw for _, _, pw in probs])
        torch.cuda.synchronize()
        for p, (w, o, pw) in enumerate(probs):
            single = H.lib().linear(xs[p], pw)
            torch.cuda.synchronize()
            assert torch.equal(ys[p].view(torch.int16), single.view(torch.int16))
            H.check_against_oracle(ys[p], xbits[p], wlc.dtype, o, wlc.group)
        for m in mats:
            H.drop((cfg, m))
