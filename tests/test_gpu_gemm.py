"""GPU parity of the matrix-core kernels (w4a16_gemm): the small-batch kernel
(M <= 32, weights streamed through registers, x in 16-row tiles) and the
LDS-tiled kernel (larger M, three tile shapes). Every output within
2e-3 * sum|x * w_hat| + 1e-5 (+ the output rounding) of the fp64 oracle, plus
exact special cases."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _gemm(x_bits, dtype, pw):
    import torch
    y = H.lib().gemm(H.to_device_bits(x_bits, dtype), pw)
    torch.cuda.synchronize()
    return y


# (N, K, group): tiny, ragged K (K % 128 = 32, 96, 64: a partial last column
# of 1, 3 or 2 chunks; K % 64 = 32: a last step of one chunk), N with a short
# last 16-row block (N % 16 = 8) and N not a multiple of the 256-wide tile.
SHAPES = [(8, 32, 32), (72, 160, 32), (200, 96, 32), (136, 256, 64), (264, 320, 64), (328, 640, 128),
          (1000, 1024, 64), (4104, 4096, 128), (520, 8192, 32)]
SKINNY_M = [1, 2, 5, 16, 17, 32]
TILED_M = [33, 37, 64, 100, 128, 129, 256, 300, 520]


def _small(N, K, group):
    return H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", SKINNY_M + TILED_M)
def test_gemm_small_shapes(N, K, group, dtype, M):
    if N * K >= 4096 * 4096 and M in (5, 17, 64, 100, 128, 129, 520):
        pytest.skip("covered by the other batch sizes at this shape")
    w, o, pw = _small(N, K, group)
    x = wl.random_activations(N * 31 + K + M, M, K, dtype)
    y = _gemm(x, dtype, pw)
    assert y.shape == (M, N)
    H.check_against_oracle(y, x, dtype, o, group)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [4, 40, 130, 300])
@pytest.mark.parametrize("N,K,group", [(72, 256, 32), (264, 320, 64), (4104, 4096, 128)])
def test_gemm_one_hot_is_exact(N, K, group, dtype, M):
    """Row m of x = e_{k_m} selects one dequantised weight per output:
    y[m][n] == round(w_hat[n][k_m]) bit for bit (w_hat is rounded at most once)."""
    import torch
    w, o, pw = _small(N, K, group)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    ks = (np.arange(M) * 7919 + 3) % K
    ks[0], ks[-1] = 0, K - 1
    x32 = np.zeros((M, K), dtype=np.float32)
    x32[np.arange(M), ks] = 1.0
    y = _gemm(wl.to_16bit(x32, dtype), dtype, pw)
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    want = ref.out_round_bits(w_hat[:, ks].T, dtype)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [3, 50])
def test_gemm_zero_input_and_linearity(M):
    import torch
    N, K, group = 328, 640, 128
    w, o, pw = _small(N, K, group)
    x0 = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    assert torch.count_nonzero(H.lib().gemm(x0, pw)).item() == 0
    x = H.to_device_bits(wl.random_activations(5 + M, M, K, "f16"), "f16")
    y1 = H.lib().gemm(x, pw).float()
    y2 = H.lib().gemm(x * 2, pw).float()
    normal = y1.abs() >= 2.0 ** -13
    assert torch.equal(y2[normal], 2 * y1[normal])


@pytest.mark.parametrize("M", [1, 16, 300])
def test_gemm_rows_are_independent(M):
    """Row m of y depends on row m of x only: the same row gives the same bits
    whatever the other rows and the batch size (no cross-row mixing)."""
    import torch
    N, K, group = 1000, 1024, 64
    w, o, pw = _small(N, K, group)
    xb = wl.random_activations(77, M, K, "bf16")
    y = H.lib().gemm(H.to_device_bits(xb, "bf16"), pw)
    y_last = H.lib().gemm(H.to_device_bits(xb[-1:], "bf16"), pw)
    torch.cuda.synchronize()
    if M <= 16:
        assert torch.equal(y[-1:].view(torch.int16), y_last.view(torch.int16))
    H.check_against_oracle(y_last, xb[-1:], "bf16", o, group)


def test_gemm_bitwise_repeatable_and_stream():
    import torch
    N, K, group = 4104, 4096, 128
    w, o, pw = _small(N, K, group)
    for M in (8, 300):
        x = H.to_device_bits(wl.random_activations(9 + M, M, K, "bf16"), "bf16")
        ys = [H.lib().gemm(x, pw) for _ in range(3)]
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            ys.append(H.lib().gemm(x, pw, stream=s))
        s.synchronize()
        torch.cuda.synchronize()
        for y in ys[1:]:
            assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


def test_linear_dispatch_matches_kernels():
    """w4a16_linear picks a kernel by M; its output is that kernel's, bit for bit."""
    import torch
    N, K, group = 1000, 1024, 64
    w, o, pw = _small(N, K, group)
    for M in (1, 2, 3, 16, 17, 32, 33, 128, 129, 300):
        x = H.to_device_bits(wl.random_activations(M, M, K, "f16"), "f16")
        y = H.lib().linear(x, pw)
        ref_fn = H.lib().gemv if H.lib().linear_kernel(M, N, K, group) == "gemv" else H.lib().gemm
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_fn(x, pw).view(torch.int16)), M


@pytest.mark.slow
@pytest.mark.parametrize("cfg,mat", [(3, 0), (5, 0)])
def test_gemm_full_size_decode_batches(cfg, mat):
    wlc = wl.WORKLOADS[cfg]
    group = wlc.group
    w, o, pw = H.prepared((cfg, mat), lambda: wl.weights(cfg, mat), group)
    for M in wlc.ms:
        x = wl.activations(cfg, mat, M)
        y = _gemm(x, wlc.dtype, pw)
        H.check_against_oracle(y, x, wlc.dtype, o, group)


@pytest.mark.slow
@pytest.mark.parametrize("fn", ["gemm", "linear"])
def test_gemm_full_size_prefill_every_output(fn):
    """The prefill configuration at its full size (M = 2048, N = 13824,
    K = 5120, bf16): every one of the 28.3 M outputs against the oracle."""
    import torch
    cfg, mat = 4, 0
    wlc = wl.WORKLOADS[cfg]
    group = wlc.group
    w, o, pw = H.prepared((cfg, mat), lambda: wl.weights(cfg, mat), group)
    M = wlc.ms[0]
    x = wl.activations(cfg, mat, M)
    y = getattr(H.lib(), fn)(H.to_device_bits(x, wlc.dtype), pw)
    torch.cuda.synchronize()
    H.check_every_output(y, x, wlc.dtype, o, group)


@pytest.mark.slow
def test_gemm_full_size_prefill_sampled_columns():
    """The prefill configuration at its full size: every row, on 320 output
    columns spread over all tiles (first and last tile included)."""
    cfg, mat = 4, 0
    wlc = wl.WORKLOADS[cfg]
    group = wlc.group
    w, o, pw = H.prepared((cfg, mat), lambda: wl.weights(cfg, mat), group)
    N = wlc.matrices[mat].N
    rng = np.random.default_rng(4)
    cols = np.unique(np.concatenate([np.arange(32), N - 32 + np.arange(32),
                                     rng.choice(N, 256, replace=False)]))
    M = wlc.ms[0]
    x = wl.activations(cfg, mat, M)
    y = _gemm(x, wlc.dtype, pw)
    H.check_against_oracle(y, x, wlc.dtype, o, group, cols=cols)
    H.drop((cfg, mat))


@pytest.mark.parametrize("M", [1, 5, 40, 300])
def test_linear_run_each_kernel(M):
    """w4a16_linear_run_fmt: every kernel that takes the shape gives a result
    within the bar of the oracle, the bits of w4a16_linear where the dispatch
    picks the same kernel; the decode kernel refuses M > 8 and an unknown
    kernel number is refused."""
    import torch
    w4 = H.lib()
    N, K, group = 520, 2048, 64
    w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
    xb = wl.random_activations(M + 77, M, K, "bf16")
    x = H.to_device_bits(xb, "bf16")
    y_lin = w4.linear(x, pw)
    chosen = w4.linear_kernel(M, N, K, group, torch.bfloat16)
    for kname in (["gemv"] if M <= 8 else []) + ["small_batch", "tiled"]:
        y = w4.linear_run(kname, x, pw)
        torch.cuda.synchronize()
        H.check_against_oracle(y, xb, "bf16", o, group)
        if kname == chosen:
            assert torch.equal(y.view(torch.int16), y_lin.view(torch.int16)), kname
    if M > 8:
        with pytest.raises(w4.W4A16Error):
            w4.linear_run("gemv", x, pw)
    y = torch.full((M, N), 1.0, dtype=torch.bfloat16, device="cuda")
    st = w4.raw().w4a16_linear_run_fmt(7, x.data_ptr(), 1, pw.qweight.data_ptr(), pw.scales.data_ptr(),
                                       pw.zeros_ptr(), y.data_ptr(), M, N, K, group, 0, None, 0, None)
    assert st == 1
    torch.cuda.synchronize()
    assert bool((y == 1.0).all())
