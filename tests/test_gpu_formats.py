"""GPU parity of the weight-format variants: symmetric 4-bit (sym4), symmetric
8-bit (sym8, W8A16), group 256 (all three formats) and the K-quant-style
256-weight super-blocks (kq4). The packed bytes,
scales and canonical view are bit-identical to the oracle's; every product is
within 2e-3 * sum|x * w_hat| + 1e-5 (+ the output rounding) of the fp64
oracle, on each kernel (GEMV, small-batch matrix-core, tiled matrix-core)."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu

FORMATS = ["asym4", "sym4", "sym8"]

# (N, K, group): ragged N (N % 16 = 8), partial last column (K % 128 = 32 / 64),
# group 256 with an odd number of groups, several tiles of the large-M kernel
SHAPES = [(8, 32, 32), (8, 256, 256), (72, 160, 32), (136, 320, 64), (328, 640, 128), (264, 768, 256),
          (1000, 1024, 256), (520, 2048, 128)]


def _prep(N, K, group, fmt):
    return H.prepared(("fmt", N, K, group), lambda: wl.random_weights(N * 3 + K + group, N, K), group, fmt)


def _check_packed(o, pw):
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(pw.qweight.cpu().numpy(), o["qweight"]), "qweight differs"
    s = pw.scales.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(s, o["scales_dev"]), "scales differ"
    if o["zeros_dev"] is None:
        assert pw.zeros is None
    else:
        assert np.array_equal(pw.zeros.cpu().numpy().view(np.uint32), o["zeros_dev"]), "zeros differ"
    codes, s_out, z_out = H.lib().unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), o["codes"])
    assert np.array_equal(s_out.cpu().numpy().view(np.uint16), o["s_bits"])
    assert np.array_equal(z_out.cpu().numpy(), o["zeros"])


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,K,group", SHAPES)
def test_pack_formats_bit_exact(N, K, group, fmt):
    w, o, pw = _prep(N, K, group, fmt)
    _check_packed(o, pw)
    q, s, z = H.lib().packed_bytes(N, K, group, fmt)
    assert (q, s, z) == (o["qweight"].size, 2 * o["scales_dev"].size,
                         0 if o["zeros_dev"] is None else 4 * o["zeros_dev"].size)


@pytest.mark.parametrize("fmt", ["sym4", "sym8"])
def test_pack_symmetric_edges(fmt):
    N, K, group = 16, 256, 64
    s = 2.0 ** -5
    qmax = 7 if fmt == "sym4" else 127
    j = np.arange(-qmax, qmax)[: group - 1]
    row = np.zeros(K, dtype=np.float64)
    row[0] = qmax * s                                    # max|w| = qmax * s: scale exactly s
    row[1:1 + j.size] = (j + 0.5) * s                    # exact ties inside the first group
    w = np.tile(row.astype(np.float32), (N, 1))
    w[1] = 0.0                                           # all-zero row: scale 2^-24, code qmax + 1
    w[2] = -1e-12                                        # scale underflows fp16
    w[3, :group] = np.float32(-2.0 ** 17)                # near the documented |w| bound
    w[4] = np.float32(1.5e-39)                           # fp32 subnormals
    o = H.oracle_pack(w, group, fmt)
    _check_packed(o, H.gpu_pack(w, group, fmt))


def _run(kernel, x_bits, dtype, pw):
    import torch
    fn = {"gemv": H.lib().gemv, "gemm": H.lib().gemm, "linear": H.lib().linear}[kernel]
    y = fn(H.to_device_bits(x_bits, dtype), pw)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kernel,M", [("gemv", 1), ("gemv", 3), ("gemm", 1), ("gemm", 17), ("gemm", 100),
                                      ("gemm", 300), ("linear", 2)])
def test_format_products_match_oracle(N, K, group, fmt, dtype, kernel, M):
    w, o, pw = _prep(N, K, group, fmt)
    x = wl.random_activations(N + K + M + len(fmt), M, K, dtype)
    y = _run(kernel, x, dtype, pw)
    assert y.shape == (M, N)
    H.check_against_oracle(y, x, dtype, o, group)


@pytest.mark.parametrize("fmt", ["sym4", "sym8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 4, 40, 300])
def test_format_one_hot_is_exact(fmt, dtype, M):
    """Row m of x = e_{k_m}: y[m][n] == round(w_hat[n][k_m]) bit for bit, on
    every kernel M reaches (GEMV for M = 1 and 4, small-batch and tiled GEMM)."""
    import torch
    N, K, group = 264, 768, 256
    w, o, pw = _prep(N, K, group, fmt)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    ks = (np.arange(M) * 7919 + 5) % K
    ks[0], ks[-1] = 0, K - 1
    x32 = np.zeros((M, K), dtype=np.float32)
    x32[np.arange(M), ks] = 1.0
    want = ref.out_round_bits(w_hat[:, ks].T, dtype)
    kernels = ["gemm", "linear"] + (["gemv"] if M <= 8 else [])
    for kernel in kernels:
        y = _run(kernel, wl.to_16bit(x32, dtype), dtype, pw)
        got = y.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want), kernel


@pytest.mark.parametrize("fmt", ["sym4", "sym8"])
@pytest.mark.parametrize("M", [1, 16, 40])
def test_format_grouped_launch_matches_single(fmt, M):
    import torch
    K, group = 1024, 128
    Ns = (1000, 136)
    pws, os_ = [], []
    for i, N in enumerate(Ns):
        w, o, pw = H.prepared(("fmt-group", N, K, group), lambda N=N: wl.random_weights(400 + N, N, K), group, fmt)
        pws.append(pw)
        os_.append(o)
    x = wl.random_activations(17 + M, M, K, "bf16")
    xd = H.to_device_bits(x, "bf16")
    ys = H.lib().linear_group([xd, xd], pws)
    torch.cuda.synchronize()
    for y, pw, o in zip(ys, pws, os_):
        single = H.lib().linear(xd, pw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), single.view(torch.int16))
        H.check_against_oracle(y, x, "bf16", o, group)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["sym4", "sym8"])
def test_format_full_size_decode_and_prefill(fmt):
    """The 4096 x 4096 decode matrix (group 128) at M = 1 and 16 in full, and the
    5120 x 13824 prefill matrix at M = 2048 on sampled columns."""
    w, o, pw = H.prepared(("fmt-full", 1), lambda: wl.weights(1, 0), 128, fmt)
    for M, dtype in ((1, "f16"), (16, "f16")):
        x = wl.activations(1, 0, M) if M == 1 else wl.random_activations(99, M, 4096, dtype)
        H.check_against_oracle(_run("linear", x, dtype, pw), x, dtype, o, 128)
    H.drop((("fmt-full", 1), fmt))
    w, o, pw = H.prepared(("fmt-full", 4), lambda: wl.weights(4, 0), 128, fmt)
    N = w.shape[0]
    cols = np.unique(np.concatenate([np.arange(16), N - 16 + np.arange(16),
                                     np.random.default_rng(3).choice(N, 96, replace=False)]))
    x = wl.activations(4, 0, 2048)
    H.check_against_oracle(_run("linear", x, "bf16", pw), x, "bf16", o, 128, cols=cols)
    H.drop((("fmt-full", 4), fmt))


# ---------------------------------------------------------------------------
# K-quant-style super-blocks (kq4, group 256)
# ---------------------------------------------------------------------------

KQ_SHAPES = [(8, 256), (72, 256), (264, 768), (1000, 1024), (520, 2048)]


def _prep_kq(N, K):
    return H.prepared(("kq", N, K), lambda: wl.random_weights(N * 5 + K, N, K), 256, "kq4")


@pytest.mark.parametrize("N,K", KQ_SHAPES)
def test_kq4_pack_bit_exact(N, K):
    import torch
    w, o, pw = _prep_kq(N, K)
    torch.cuda.synchronize()
    assert np.array_equal(pw.qweight.cpu().numpy(), o["qweight"]), "codes differ"
    rec = pw.scales.cpu().view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(rec, o["records"]), "super-block records differ"
    codes, _, _ = H.lib().unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), o["codes"])
    assert H.lib().packed_bytes(N, K, 256, "kq4") == (N * K // 2, 16 * (K // 256) * N, 0)


def test_kq4_pack_edges():
    N, K = 24, 512
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    w[0] = 0.0                                    # all-zero super-blocks
    w[1] = np.abs(w[1])                           # no minimum
    w[2] = -np.abs(w[2])                          # no positive part
    w[3, :256] = 1e-12                            # scales underflow fp16
    w[4, :32] = np.float32(2.0 ** 17)             # one large sub-block
    w[5, :] = -0.0                                # negative zeros
    o = H.oracle_pack(w, 256, "kq4")
    pw = H.gpu_pack(w, 256, "kq4")
    import torch
    assert np.array_equal(pw.qweight.cpu().numpy(), o["qweight"])
    assert np.array_equal(pw.scales.cpu().view(torch.int32).numpy().view(np.uint32), o["records"])


@pytest.mark.parametrize("N,K", KQ_SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kernel,M", [("gemv", 1), ("gemv", 5), ("gemm", 1), ("gemm", 17), ("gemm", 100),
                                      ("gemm", 300), ("linear", 2)])
def test_kq4_products_match_oracle(N, K, dtype, kernel, M):
    w, o, pw = _prep_kq(N, K)
    x = wl.random_activations(N + K + M + 7, M, K, dtype)
    y = _run(kernel, x, dtype, pw)
    H.check_against_oracle(y, x, dtype, o, 256)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 4, 40, 300])
def test_kq4_one_hot(dtype, M):
    """One-hot rows select one rebuilt weight w_hat = S q - M: every kernel forms
    it with one fp32 fma and rounds it once more to 16 bit, as the oracle's
    output rounding does, so the result is bit-exact on all three kernels."""
    import torch
    N, K = 264, 768
    w, o, pw = _prep_kq(N, K)
    w_hat = ref.dequantize_kquant(o["codes"], *o["kq"])
    ks = (np.arange(M) * 7919 + 11) % K
    ks[0], ks[-1] = 0, K - 1
    x32 = np.zeros((M, K), dtype=np.float32)
    x32[np.arange(M), ks] = 1.0
    want = ref.out_round_bits(w_hat[:, ks].T, dtype)
    kernels = ["gemm", "linear"] + (["gemv"] if M <= 8 else [])
    for kernel in kernels:
        y = _run(kernel, wl.to_16bit(x32, dtype), dtype, pw)
        got = y.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want), kernel


def test_kq4_quality_report():
    import torch
    N, K = 520, 2048
    w, o, pw = _prep_kq(N, K)
    got = H.lib().quant_error(torch.from_numpy(w).cuda(), pw)
    w_hat = ref.dequantize_kquant(o["codes"], *o["kq"])
    sums = ref.quant_error_sums(w, w_hat)
    mse, snr, cos, mx = ref.quant_error_stats(sums, w_hat.size)
    assert got["max_err"] == mx
    assert abs(got["mse"] - mse) <= 1e-12 * mse and abs(got["snr_db"] - snr) <= 1e-9 and abs(got["cos"] - cos) <= 1e-12


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["sym8", "kq4"])
def test_format_full_size_70b_down(fmt):
    """The 70B down projection (K = 28672, N = 8192) packed as W8A16 and as
    K-quant super-blocks, M = 1 and 8, every output against the oracle."""
    group = 256 if fmt == "kq4" else 32
    w, o, pw = H.prepared(("fmt-full", 5), lambda: wl.weights(5, 0), group, fmt)
    for M in (1, 8):
        x = wl.activations(5, 0, M)
        H.check_against_oracle(_run("linear", x, "f16", pw), x, "f16", o, group)
    H.drop((("fmt-full", 5), fmt))


@pytest.mark.parametrize("M", [1, 16])
def test_kq4_grouped_launch_matches_single(M):
    import torch
    K = 1024
    pws, os_ = [], []
    for N in (1000, 136):
        w, o, pw = H.prepared(("kq-group", N, K), lambda N=N: wl.random_weights(900 + N, N, K), 256, "kq4")
        pws.append(pw)
        os_.append(o)
    x = wl.random_activations(5 + M, M, K, "f16")
    xd = H.to_device_bits(x, "f16")
    ys = H.lib().linear_group([xd, xd], pws)
    torch.cuda.synchronize()
    for y, pw, o in zip(ys, pws, os_):
        single = H.lib().linear(xd, pw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), single.view(torch.int16))
        H.check_against_oracle(y, x, "f16", o, 256)
