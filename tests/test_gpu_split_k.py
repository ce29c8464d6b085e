"""GPU parity of the tiled GEMM's K split: when its tiles fill at most half of
the compute units (mid-size batches), each tile's 128-weight columns are split
over S workgroups, each leaving an fp32 partial tile in the workspace; the last
to arrive adds the S partials in split order. Outputs within the bar of the
oracle (R19) on every output, one-hot inputs bit-exact, repeat calls and graph
replays bit-identical, any workspace contents accepted, a short workspace
refused. The tiled kernel is run by choice (w4a16_linear_run_fmt), so the
split is tested at batch sizes where w4a16_linear may pick another kernel."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu

# (M, N, K, group) on 256 compute units, 64-row tiles unless stated: 1 x 4 tiles split 4
# ways; a ragged M, N and K (N % 16 = 8, K % 128 = 32: 68 tiles split 2 ways,
# the last split holding the partial last column); group 256 (one metadata
# slot per two columns, 16 tiles split 8 ways); 20 tiles split 6 ways; the
# mid-batch QKV shape (M = 64: 60 tiles of 64 rows split 4 ways; M = 128: 60
# tiles of 128 rows split 4 ways)
SPLIT_SHAPES = [(37, 1000, 2048, 64), (200, 4104, 1056, 32), (100, 2048, 4096, 256), (300, 1024, 3072, 128),
                (64, 15360, 5120, 128), (128, 15360, 5120, 128)]


def _prep(N, K, group, fmt="asym4"):
    return H.prepared(("splitk", N, K, group), lambda: wl.random_weights(N * 5 + K, N, K), group, fmt)


FMT_CODE = {"asym4": 0, "sym4": 1, "sym8": 2, "kq4": 3}


def _kernel_ws(M, N, K, group, fmt="asym4"):
    """w4a16_kernel_workspace_bytes of the tiled kernel (kernel 2)."""
    import ctypes
    nb = ctypes.c_size_t()
    st = H.lib().raw().w4a16_kernel_workspace_bytes(2, M, N, K, group, FMT_CODE[fmt], ctypes.byref(nb))
    assert st == 0
    return nb.value


@pytest.mark.parametrize("M,N,K,group", SPLIT_SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_k_matches_oracle_everywhere(M, N, K, group, dtype):
    import torch
    assert _kernel_ws(M, N, K, group) > 0, "shape expected to take the K split"
    w, o, pw = _prep(N, K, group)
    x = wl.random_activations(M + N + K, M, K, dtype)
    y = H.lib().linear_run("tiled", H.to_device_bits(x, dtype), pw)
    torch.cuda.synchronize()
    if N * M <= 2 * 10 ** 6:
        H.check_every_output(y, x, dtype, o, group)
    else:
        rng = np.random.default_rng(M + N)
        H.check_against_oracle(y, x, dtype, o, group,
                               cols=np.unique(np.concatenate([np.arange(256), rng.choice(N, 512, replace=False)])))


@pytest.mark.parametrize("fmt", ["sym4", "sym8", "kq4"])
def test_split_k_formats(fmt):
    import torch
    M, N, K = 96, 2048, 4096
    group = 256 if fmt == "kq4" else 128
    assert _kernel_ws(M, N, K, group, fmt) > 0
    w, o, pw = _prep(N, K, group, fmt)
    x = wl.random_activations(29, M, K, "bf16")
    y = H.lib().linear_run("tiled", H.to_device_bits(x, "bf16"), pw)
    torch.cuda.synchronize()
    H.check_every_output(y, x, "bf16", o, group)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_k_one_hot_is_exact(dtype):
    """One-hot rows: every split but one adds an exact zero, so the sum is
    round(w_hat) bit for bit."""
    import torch
    M, N, K, group = 64, 2048, 4096, 128
    w, o, pw = _prep(N, K, group)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    ks = (np.arange(M) * 7919 + 3) % K
    x32 = np.zeros((M, K), dtype=np.float32)
    x32[np.arange(M), ks] = 1.0
    y = H.lib().linear_run("tiled", H.to_device_bits(wl.to_16bit(x32, dtype), dtype), pw)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    want = ref.out_round_bits(w_hat[:, ks].T, dtype)
    assert np.array_equal(got, want)


def test_split_k_repeatable_any_workspace_and_graph_replay():
    """The same call three times (once on a workspace of random bytes) and
    three replays of a captured graph give the same bits: the arrival counters
    carry a per-launch token and are cleared by the last arrival."""
    import torch
    w4 = H.lib()
    M, N, K, group = 128, 4096, 5120, 128
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(17, M, K, "f16"), "f16")
    nbytes = _kernel_ws(M, N, K, group)
    assert nbytes > 0
    ws = w4.Workspace(torch.device("cuda"))
    first = w4.linear_run("tiled", x, pw, workspace=ws)
    again = w4.linear_run("tiled", x, pw, workspace=ws)
    buf = ws.get(nbytes)
    buf.copy_(torch.randint(0, 256, (buf.numel(),), dtype=torch.uint8, device="cuda"))
    junk = w4.linear_run("tiled", x, pw, workspace=ws)
    torch.cuda.synchronize()
    for y in (again, junk):
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))
    out = torch.empty_like(first)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    w4.linear_run("tiled", x, pw, out=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.linear_run("tiled", x, pw, out=out, workspace=ws, stream=s)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    H.check_against_oracle(first, wl.random_activations(17, M, K, "f16"), "f16", o, group, cols=np.arange(0, N, 37))


def test_split_k_short_workspace_refused_and_plan_limits():
    """One byte less than w4a16_kernel_workspace_bytes is refused before
    anything runs; grids that fill more than half the compute units get no
    split (no workspace)."""
    import torch
    w4 = H.lib()
    M, N, K, group = 64, 2048, 4096, 128
    w, o, pw = _prep(N, K, group)
    nbytes = _kernel_ws(M, N, K, group)
    assert nbytes > 0
    x = H.to_device_bits(wl.random_activations(3, M, K, "f16"), "f16")
    y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = w4.raw().w4a16_linear_run_fmt(2, x.data_ptr(), 0, pw.qweight.data_ptr(), pw.scales.data_ptr(),
                                       pw.zeros_ptr(), y.data_ptr(), M, N, K, group, 0, ws.data_ptr(), nbytes - 1,
                                       None)
    assert st == 4   # W4A16_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # 64-row tiles: 4 x 33 = 132 tiles on 256 compute units, more than half: whole tiles
    assert _kernel_ws(256, 8448, 512, 128) == 0
