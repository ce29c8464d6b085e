"""GPU parity of the decode GEMV (w4a16_gemv): every output within
2e-3 * sum|x * w_hat| + 1e-5 of the fp64 oracle, plus exact special cases."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _run(fn, x_bits, dtype, pw):
    import torch
    y = fn(H.to_device_bits(x_bits, dtype), pw)
    torch.cuda.synchronize()
    return y


def _dec_lds_per_wave(mt, ncol, group):
    """LDS bytes of one decode wave (4-bit zero-point format): activations,
    activation sums, the 16 rows' scales and zero-point words, 16 spare bytes."""
    upc = 1 if group >= 128 else 128 // group
    meta_row = ncol if group >= 256 else ncol * (128 // group) * 2
    zwords = (ncol // 2 + 7) // 8 if group >= 256 else (ncol * (128 // group) + 7) // 8
    return mt * ncol * 256 + mt * ncol * upc * 32 + 16 * meta_row + 16 * zwords * 4 + 16


def gemv_accepts(M, K, dtype, group=32):
    """The decode kernel's range: M <= 8 and all of K in one workgroup of at
    most 16 waves (8 columns of 128 weights per wave, or 16 for one or two
    activation rows), its LDS within gfx950's 160 KiB per workgroup."""
    if not 1 <= M <= 8:
        return False
    T = -(-(K // 32) // 4)
    mt = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
    if -(-T // 8) <= 16:
        ncol = 8
    elif mt <= 2 and -(-T // 16) <= 16:
        ncol = 16
    else:
        return False
    return -(-T // ncol) * _dec_lds_per_wave(mt, ncol, group) <= 160 * 1024


SMALL = [(8, 32, 32), (72, 64, 32), (200, 96, 32), (136, 256, 64), (64, 384, 128), (328, 640, 128),
         (1000, 1024, 64), (4104, 4096, 128), (520, 8192, 32), (40, 160, 32), (24, 1120, 32),
         (48, 16384, 128), (24, 32768, 64)]


@pytest.mark.parametrize("N,K,group", SMALL)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_gemv_small_shapes(N, K, group, dtype, M):
    w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
    x = wl.random_activations(N * 31 + K + M, M, K, dtype)
    if not gemv_accepts(M, K, dtype, group):
        # outside the decode kernel's range: an invalid-argument error, no launch
        with pytest.raises(H.lib().W4A16Error):
            _run(H.lib().gemv, x, dtype, pw)
        return
    y = _run(H.lib().gemv, x, dtype, pw)
    assert y.shape == (M, N)
    H.check_against_oracle(y, x, dtype, o, group)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,K,group", [(72, 256, 32), (200, 512, 128), (4104, 4096, 128)])
def test_gemv_one_hot_is_exact(N, K, group, dtype):
    """x = e_k selects one dequantised weight per output: y[n] == round(w_hat[n][k])."""
    w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    for k in (0, group - 1, K // 2 + 3, K - 1):
        x32 = np.zeros((1, K), dtype=np.float32)
        x32[0, k] = 1.0
        xb = wl.to_16bit(x32, dtype)
        y = _run(H.lib().gemv, xb, dtype, pw)
        got = y.cpu().view(__import__("torch").int16).numpy().view(np.uint16)[0]
        want = ref.out_round_bits(w_hat[:, k], dtype)
        assert np.array_equal(got, want), k


def test_gemv_zero_input_and_linearity():
    import torch
    N, K, group = 328, 640, 128
    w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
    x0 = torch.zeros((2, K), dtype=torch.float16, device="cuda")
    y0 = H.lib().gemv(x0, pw)
    assert torch.count_nonzero(y0).item() == 0
    # scaling x by 2 scales y by 2 exactly (powers of two commute with rounding)
    xb = wl.random_activations(3, 2, K, "f16")
    x = H.to_device_bits(xb, "f16")
    y1 = H.lib().gemv(x, pw).float()
    y2 = H.lib().gemv(x * 2, pw).float()
    normal = y1.abs() >= 2.0 ** -13      # away from fp16 subnormals, where rounding is absolute
    assert torch.equal(y2[normal], 2 * y1[normal])


def test_gemv_bitwise_repeatable_and_stream():
    import torch
    N, K, group = 4104, 4096, 128
    w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
    x = H.to_device_bits(wl.random_activations(9, 1, K, "f16"), "f16")
    ys = [H.lib().gemv(x, pw) for _ in range(5)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ys.append(H.lib().gemv(x, pw, stream=s))
    s.synchronize()
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


@pytest.mark.slow
@pytest.mark.parametrize("cfg,mat", [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3), (2, 4), (2, 5), (2, 6), (5, 0)])
def test_gemv_full_size_configs(cfg, mat):
    wlc = wl.WORKLOADS[cfg]
    group = wlc.group
    w, o, pw = H.prepared((cfg, mat), lambda: wl.weights(cfg, mat), group)
    for M in wlc.ms:
        if not gemv_accepts(M, wlc.matrices[mat].K, wlc.dtype, group):
            continue
        x = wl.activations(cfg, mat, M)
        y = _run(H.lib().gemv, x, wlc.dtype, pw)
        H.check_against_oracle(y, x, wlc.dtype, o, group)
    if cfg == 2:
        H.drop((cfg, mat))


def test_workspace_reused_across_shapes():
    """One workspace serves consecutive calls of different shapes (counters stay zeroed)."""
    shapes = [(1000, 1024, 64), (4104, 4096, 128), (136, 256, 64), (8200, 2048, 32), (4104, 4096, 128)]
    ws = H.lib().Workspace()
    for N, K, group in shapes:
        w, o, pw = H.prepared(("small", N, K, group), lambda: wl.random_weights(N + K, N, K), group)
        for M in (1, 3):
            x = wl.random_activations(N + M, M, K, "f16")
            import torch
            y = H.lib().gemv(H.to_device_bits(x, "f16"), pw, workspace=ws)
            torch.cuda.synchronize()
            H.check_against_oracle(y, x, "f16", o, group)
