"""Edge cases of the product calls through the binding: an empty batch (M = 0)
returns an empty result and enqueues nothing, and the binding refuses outputs
and packed buffers that do not match the shape before any launch."""
import numpy as np
import pytest

import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu

N, K, GROUP = 264, 768, 128


def _prep(fmt="asym4"):
    return H.prepared(("edges", fmt), lambda: wl.random_weights(23, N, K), GROUP, fmt)


@pytest.mark.parametrize("fmt", ["asym4", "sym8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_empty_batch(fmt, dtype):
    import torch
    w4 = H.lib()
    w, o, pw = _prep(fmt)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    x0 = torch.empty((0, K), dtype=tdt, device="cuda")
    for fn in (w4.gemv, w4.gemm, w4.linear):
        y = fn(x0, pw)
        assert y.shape == (0, N) and y.dtype == tdt
    ys = w4.linear_group([x0, x0], [pw, pw])
    assert [tuple(y.shape) for y in ys] == [(0, N), (0, N)]
    m = torch.ones(K, dtype=torch.float32, device="cuda")
    assert w4.linear_awq(x0, m, pw).shape == (0, N)
    assert w4.scale_activations(x0, m).shape == (0, K)
    # a call after the empty ones is unaffected
    x = wl.random_activations(5, 3, K, dtype)
    y = w4.linear(H.to_device_bits(x, dtype), pw)
    torch.cuda.synchronize()
    H.check_against_oracle(y, x, dtype, o, GROUP)


def test_binding_rejects_mismatched_outputs():
    import torch
    w4 = H.lib()
    w, o, pw = _prep()
    x = H.to_device_bits(wl.random_activations(6, 2, K, "f16"), "f16")
    sentinel = torch.full((2, N + 8), 7.0, dtype=torch.float16, device="cuda")
    bad = [torch.empty((2, N - 8), dtype=torch.float16, device="cuda"),      # too small
           torch.empty((2, N), dtype=torch.bfloat16, device="cuda"),         # other type
           torch.empty((3, N), dtype=torch.float16, device="cuda"),          # other M
           sentinel[:, :N]]                                                  # not contiguous
    for out in bad:
        for fn in (w4.gemv, w4.gemm, w4.linear):
            with pytest.raises(ValueError):
                fn(x, pw, out=out)
        with pytest.raises(ValueError):
            w4.linear_group([x], [pw], outs=[out])
    with pytest.raises(ValueError):
        w4.linear_group([x, x], [pw, pw], outs=[torch.empty((2, N), dtype=torch.float16, device="cuda")])
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_binding_rejects_short_packed_buffers():
    import torch
    w4 = H.lib()
    w, o, pw = _prep()
    with pytest.raises(ValueError):
        w4.PackedWeight(pw.qweight[:-16], pw.scales, pw.zeros, N, K, GROUP)
    with pytest.raises(ValueError):
        w4.PackedWeight(pw.qweight, pw.scales[:-8], pw.zeros, N, K, GROUP)
    with pytest.raises(ValueError):
        w4.PackedWeight(pw.qweight, pw.scales, None, N, K, GROUP)                  # asym4 needs zeros
    with pytest.raises(ValueError):
        w4.PackedWeight(pw.qweight, pw.scales, pw.zeros, N + 8, K, GROUP)          # shape larger than the data
    with pytest.raises(ValueError):
        w4.PackedWeight(pw.qweight.cpu(), pw.scales, pw.zeros, N, K, GROUP)        # host memory
    ok = w4.PackedWeight(pw.qweight, pw.scales, pw.zeros, N, K, GROUP)
    x = H.to_device_bits(wl.random_activations(8, 1, K, "f16"), "f16")
    y0, y1 = w4.linear(x, pw), w4.linear(x, ok)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert np.isfinite(y0.float().cpu().numpy()).all()
