"""GPU parity of the decode path for one activation row and long K (sixteen
128-weight columns per wave, K > 16384): there the decode kernel keeps the
activations in registers and broadcasts each chunk's slice across a row of
lanes (decode_bcast_kernel). It forms the same sums in the same order as the
kernel that stages the activations in LDS, which the grouped call still runs,
so the two must agree bit for bit; both must be within the bar of the fp64
oracle on every output."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu

# (N, K, group): 129 columns (9 waves, the last with one column), ragged last
# row block, every group size, metadata through LDS (32, 64) and in registers
# (128, 256); the 70B down projection's K
SHAPES = [(40, 16512, 32), (264, 20480, 64), (136, 24576, 128), (72, 28672, 256), (1032, 28672, 32),
          (24, 32768, 128)]


def _threads(N, K, group, dtype, fmt="asym4"):
    import torch
    kern, wgs, thr = H.lib().linear_launch_shape(1, N, K, group,
                                                 torch.bfloat16 if dtype == "bf16" else torch.float16, fmt)
    assert kern == "gemv" and wgs == (N + 15) // 16, (kern, wgs)
    return thr


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", ["asym4", "sym4"])
def test_long_k_single_row_every_output(N, K, group, dtype, fmt):
    import torch
    T = K // 128
    assert _threads(N, K, group, dtype, fmt) == 64 * -(-T // 16), "sixteen columns per wave"
    w, o, pw = H.prepared(("long_k", N, K, group), lambda: wl.random_weights(N * 3 + K + group, N, K), group, fmt)
    xb = wl.random_activations(N + K + group, 1, K, dtype)
    x = H.to_device_bits(xb, dtype)
    y = H.lib().linear(x, pw)
    (yg,) = H.lib().linear_group([x], [pw])
    yv = H.lib().gemv(x, pw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yg.view(torch.int16)), "differs from the grouped launch"
    assert torch.equal(y.view(torch.int16), yv.view(torch.int16))
    H.check_every_output(y, xb, dtype, o, group)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_long_k_single_row_one_hot_is_exact(dtype):
    """x = e_k selects one dequantised weight per output: y[n] == round(w_hat[n][k])
    for k in the first, a middle and the last column, every wave's slice."""
    import torch
    N, K, group = 1032, 28672, 32
    w, o, pw = H.prepared(("long_k", N, K, group), lambda: wl.random_weights(N * 3 + K + group, N, K), group)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    for k in (0, 31, 2048 + 77, K // 2 + 5, K - 129, K - 1):
        x32 = np.zeros((1, K), dtype=np.float32)
        x32[0, k] = 1.0
        y = H.lib().linear(H.to_device_bits(wl.to_16bit(x32, dtype), dtype), pw)
        torch.cuda.synchronize()
        got = y.cpu().view(torch.int16).numpy().view(np.uint16)[0]
        assert np.array_equal(got, ref.out_round_bits(w_hat[:, k], dtype)), k


def test_long_k_single_row_zero_and_scaling():
    """Zero activations give exact zeros; doubling x doubles y exactly away from
    fp16 subnormals (every step of the kernel commutes with a power of two)."""
    import torch
    N, K, group = 264, 20480, 64
    w, o, pw = H.prepared(("long_k", N, K, group), lambda: wl.random_weights(N * 3 + K + group, N, K), group)
    y0 = H.lib().linear(torch.zeros((1, K), dtype=torch.float16, device="cuda"), pw)
    xb = wl.random_activations(5, 1, K, "f16")
    x = H.to_device_bits(xb, "f16")
    y1 = H.lib().linear(x, pw).float()
    y2 = H.lib().linear(x * 2, pw).float()
    torch.cuda.synchronize()
    assert torch.count_nonzero(y0).item() == 0
    normal = y1.abs() >= 2.0 ** -13
    assert torch.equal(y2[normal], 2 * y1[normal])
