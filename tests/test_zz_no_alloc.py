"""w4a16_linear_noalloc (the static-scratch variant of w4a16_linear_fmt, for
callers that cannot allocate) against w4a16_linear_fmt through the C ABI:
two stream-K calls in a row on the shared scratch, the second smaller, plus
a decode and a small-batch call; every output bit-identical to the ordinary
entry point's and within the bar of the oracle."""
import numpy as np
import pytest

import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu

W4A16_BF16 = 1


def _ordinary(x, pw, M, stream):
    import torch
    w4 = H.lib()
    nbytes = w4.workspace_bytes(M, pw.N, pw.K, pw.group)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, pw.N), dtype=x.dtype, device="cuda")
    st = w4.raw().w4a16_linear_fmt(x.data_ptr(), W4A16_BF16, pw.qweight.data_ptr(), pw.scales.data_ptr(),
                                   pw.zeros_ptr(), y.data_ptr(), M, pw.N, pw.K, pw.group, 0,
                                   ws.data_ptr() if nbytes else None, nbytes, stream.cuda_stream)
    assert st == 0, st
    return y, nbytes


def _noalloc(x, pw, M, stream):
    import torch
    w4 = H.lib()
    y = torch.full((M, pw.N), float("nan"), dtype=x.dtype, device="cuda")
    st = w4.raw().w4a16_linear_noalloc(x.data_ptr(), W4A16_BF16, pw.qweight.data_ptr(), pw.scales.data_ptr(),
                                       pw.zeros_ptr(), y.data_ptr(), M, pw.N, pw.K, pw.group, 0, stream.cuda_stream)
    assert st == 0, st
    return y


def test_noalloc_matches_linear_on_consecutive_calls():
    import torch
    w4 = H.lib()
    assert w4.raw().w4a16_init(0) == 0
    stream = torch.cuda.Stream()
    K, group = 2048, 128
    # (M, N): two stream-K splits (the second smaller, ragged M), then a decode
    # call and a small-batch call that use no scratch, then the first again
    cases = [(2048, 8448), (2000, 8448), (1, 8448), (17, 8448), (2048, 8448)]
    w, o, pw = H.prepared(("noalloc", 8448, K, group), lambda: wl.random_weights(77, 8448, K), group)
    needs = []
    for i, (M, N) in enumerate(cases):
        x = H.to_device_bits(wl.random_activations(500 + i, M, K, "bf16"), "bf16")
        with torch.cuda.stream(stream):
            y_ref, nbytes = _ordinary(x, pw, M, stream)
            y = _noalloc(x, pw, M, stream)
        stream.synchronize()
        needs.append(nbytes)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (M, N)
        cols = np.unique(np.concatenate([np.arange(16), N - 16 + np.arange(16),
                                         np.random.default_rng(i).choice(N, 96, replace=False)]))
        xb = wl.random_activations(500 + i, M, K, "bf16")
        H.check_against_oracle(y, xb, "bf16", o, group, cols=cols)
    assert needs[0] > 0 and needs[1] > 0 and needs[2] == 0 and needs[3] == 0


def test_noalloc_decode_long_k_and_split_k():
    """One activation row: the long-K decode variant (no scratch) and the
    decode kernel's K split (its partials and counters in the static scratch),
    in a row, the split twice with a smaller shape between; bit-identical to
    w4a16_linear_fmt with a workspace and within the bar on every output."""
    import torch
    w4 = H.lib()
    assert w4.raw().w4a16_init(0) == 0
    stream = torch.cuda.Stream()
    group = 128
    cases = [(40, 65536), (264, 24576), (24, 65536), (40, 65536)]
    needs = []
    for i, (N, K) in enumerate(cases):
        w, o, pw = H.prepared(("noalloc_dec", N, K, group), lambda: wl.random_weights(31 * N + K, N, K), group)
        xb = wl.random_activations(900 + i, 1, K, "bf16")
        x = H.to_device_bits(xb, "bf16")
        with torch.cuda.stream(stream):
            y_ref, nbytes = _ordinary(x, pw, 1, stream)
            y = _noalloc(x, pw, 1, stream)
        stream.synchronize()
        needs.append(nbytes)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (N, K)
        H.check_every_output(y, xb, "bf16", o, group)
    assert needs[0] > 0 and needs[1] == 0 and needs[2] > 0


def test_noalloc_rejects_bad_arguments_and_writes_nothing():
    import torch
    w4 = H.lib()
    assert w4.raw().w4a16_init(0) == 0
    K, group = 2048, 128
    w, o, pw = H.prepared(("noalloc", 8448, K, group), lambda: wl.random_weights(77, 8448, K), group)
    x = H.to_device_bits(wl.random_activations(9, 4, K, "bf16"), "bf16")
    y = torch.full((4, pw.N), 5.0, dtype=torch.bfloat16, device="cuda")
    raw = w4.raw()
    head = (x.data_ptr(), W4A16_BF16, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(), y.data_ptr())
    assert raw.w4a16_linear_noalloc(*head, 4, pw.N, K + 1, group, 0, None) == 1     # K % group != 0
    assert raw.w4a16_linear_noalloc(*head, 4, pw.N, K, 48, 0, None) == 1           # no such group
    assert raw.w4a16_linear_noalloc(*head, 4, pw.N, K, group, 9, None) == 1        # no such format
    assert raw.w4a16_linear_noalloc(*head, (1 << 24) + 1, pw.N, K, group, 0, None) == 1   # M too large
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
    with pytest.raises(ValueError):
        w4.linear_noalloc(x, pw, None)
