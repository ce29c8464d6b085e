"""GPU parity of the quality report (w4a16_quant_error) and of AWQ's run-time
activation scaling (w4a16_scale_activations, w4a16_linear_awq) against the
oracle: rounded activations bit for bit, reports to fp64 summation-order
tolerance (the largest error exactly), products within the usual bar."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _report(w, pw):
    import torch
    return H.lib().quant_error(torch.from_numpy(np.ascontiguousarray(w)).cuda(), pw)


def _check_report(got, w, o, group):
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    sums = ref.quant_error_sums(w, w_hat)
    mse, snr, cos, mx = ref.quant_error_stats(sums, w_hat.size)
    assert got["max_err"] == mx
    for key, want in zip(("sum_d2", "sum_w2", "sum_h2", "sum_wh"), sums[:4]):
        assert abs(got[key] - want) <= 1e-12 * abs(want) + 1e-300, key
    assert abs(got["mse"] - mse) <= 1e-12 * mse + 1e-300
    if np.isinf(snr):
        assert got["snr_db"] == snr
    else:
        assert abs(got["snr_db"] - snr) <= 1e-9
    assert abs(got["cos"] - cos) <= 1e-12


@pytest.mark.parametrize("fmt", ["asym4", "sym4", "sym8"])
@pytest.mark.parametrize("N,K,group", [(72, 160, 32), (328, 640, 128), (264, 768, 256), (1000, 1024, 64)])
def test_quant_error_matches_oracle(N, K, group, fmt):
    w, o, pw = H.prepared(("qe", N, K, group), lambda: wl.random_weights(7 * N + K, N, K), group, fmt)
    _check_report(_report(w, pw), w, o, group)


def test_quant_error_degenerate_matrices():
    N, K, group = 24, 256, 128
    z = np.zeros((N, K), dtype=np.float32)
    o = H.oracle_pack(z, group)
    got = _report(z, H.gpu_pack(z, group))
    assert (got["mse"], got["snr_db"], got["cos"], got["max_err"]) == (0.0, np.inf, 1.0, 0.0)
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::group], q[:, 1::group] = 0, 15
    lat = ((q - 4) * 2.0 ** -7).astype(np.float32)           # on the grid: exact
    o = H.oracle_pack(lat, group)
    got = _report(lat, H.gpu_pack(lat, group))
    assert got["sum_d2"] == 0.0 and got["snr_db"] == np.inf and got["max_err"] == 0.0
    _check_report(got, lat, o, group)


@pytest.mark.parametrize("N,K,group,fmt", [(16, 4128, 32, "asym4"),      # one row block, 33 one-column slices
                                            (40, 8288, 32, "sym8"),       # 3 row blocks (one ragged), 65 slices
                                            (9000, 1280, 256, "sym4")])   # 563 row blocks, 4 slices of 2 or 3 columns
def test_quant_error_k_slices(N, K, group, fmt):
    """The report's partial sums are taken per (row block, slice of K's
    128-weight columns): shapes at both ends of the split, ragged slices
    included, against the oracle; the device-result form (out=) gives the same
    numbers, bit-identical on repeat whatever the workspace held before."""
    import torch
    w4 = H.lib()
    w = wl.random_weights(3 * N + K, N, K)
    o, pw = H.oracle_pack(w, group, fmt), H.gpu_pack(w, group, fmt)
    wt = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    got = w4.quant_error(wt, pw)
    _check_report(got, w, o, group)
    ws = w4.Workspace("cuda")
    buf = ws.get(1 << 20)
    buf.copy_(torch.randint(0, 256, buf.shape, dtype=torch.uint8, device="cuda"))
    out = torch.full((8,), 7.0, dtype=torch.float64, device="cuda")
    for _ in range(2):
        assert w4.quant_error(wt, pw, out=out, workspace=ws) is out
        torch.cuda.synchronize()
        assert out.cpu().tolist() == [got[f] for f in w4.QUALITY_FIELDS]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 64), (3, 1000 // 8 * 8), (17, 5120), (300, 640)])
def test_scale_activations_bit_exact(dtype, M, K):
    import torch
    rng = np.random.default_rng(M + K)
    m = rng.uniform(0.02, 8.0, size=K).astype(np.float32)
    m[0] = 1.0
    m[-1] = 2.0 ** -20                                         # towards the subnormal range
    x = wl.random_activations(M * 5 + K, M, K, dtype)
    xd = H.to_device_bits(x, dtype)
    md = torch.from_numpy(m).cuda()
    got = H.lib().scale_activations(xd, md)
    torch.cuda.synchronize()
    want = ref.awq_scale_activations(x, dtype, m)
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), want)
    # in place
    H.lib().scale_activations(xd, md, out=xd)
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("fmt", ["asym4", "sym8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 4, 8, 16, 300])
def test_linear_awq(fmt, dtype, M):
    """AWQ: weights quantised after scaling 1 % of the input channels up by 8,
    activations multiplied by the reciprocals. Fused GEMV path (M <= 8) and
    pre-scale + GEMM path give the kernel's result on the pre-scaled activations
    bit for bit, and match the oracle."""
    import torch
    N, K, group = 520, 2048, 128
    rng = np.random.default_rng(9)
    a = np.ones(K, dtype=np.float32)
    a[rng.choice(K, K // 100, replace=False)] = 8.0
    m = (1.0 / a).astype(np.float32)
    w = wl.random_weights(11, N, K)
    wf = ref.awq_fold_weights(w, a)
    _, o, pw = H.prepared(("awq", N, K, group), lambda: wf, group, fmt)
    x = wl.random_activations(M + 3, M, K, dtype)
    xd = H.to_device_bits(x, dtype)
    md = torch.from_numpy(m).cuda()
    y = H.lib().linear_awq(xd, md, pw)
    xs = H.lib().scale_activations(xd, md)
    fn = H.lib().gemv if M <= 8 else H.lib().gemm
    y_pre = fn(xs, pw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_pre.view(torch.int16))
    xs_ref = ref.awq_scale_activations(x, dtype, m)
    H.check_against_oracle(y, xs_ref, dtype, o, group)


@pytest.mark.slow
def test_quant_error_full_size_decode_layer_set():
    """The quality report of every matrix of the 13B decode layer set (group 128)."""
    cfg = 2
    for mat in range(len(wl.WORKLOADS[cfg].matrices)):
        w, o, pw = H.prepared(("qe-full", mat), lambda mat=mat: wl.weights(cfg, mat), 128)
        _check_report(_report(w, pw), w, o, 128)
        H.drop(("qe-full", mat))
