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


def gemv_accepts(M, K, dtype, group=32):
    """The decode kernel's range: M <= 8 and K <= 65536 (it splits K over
    workgroups until a workgroup's LDS fits)."""
    return 1 <= M <= 8 and K <= 65536


SMALL = [(8, 32, 32), (72, 64, 32), (200, 96, 32), (136, 256, 64), (64, 384, 128), (328, 640, 128),
         (1000, 1024, 64), (4104, 4096, 128), (520, 8192, 32), (40, 160, 32), (24, 1120, 32),
         (48, 16384, 128), (24, 32768, 64), (16, 65536, 128), (40, 5152, 32), (8, 131072, 128)]


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


# (M, N, K, group) whose decode plan splits K over several workgroups per row
# block (a workgroup's activations and metadata for all of K would pass the
# LDS), ragged K and a short last row block included
SPLIT = [(1, 136, 65536, 128), (2, 1032, 28672, 32), (3, 520, 32768, 32), (5, 24, 13824, 64),
         (8, 40, 16416, 32)]


@pytest.mark.parametrize("M,N,K,group", SPLIT)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_k_decode_is_deterministic_across_workspaces_and_replays(M, N, K, group, dtype):
    """Split-K decode: the same bits from a fresh workspace, from one whose
    counters and partials hold junk (random bytes, then small integers), and
    from every replay of a captured graph; every output within the bar."""
    import torch
    w4 = H.lib()
    assert w4.workspace_bytes(M, N, K, group) > 0   # the plan splits K
    w, o, pw = H.prepared(("split", N, K, group), lambda: wl.random_weights(N * 7 + K, N, K), group)
    for _ in (0,):
        xb = wl.random_activations(N + 5 * M, M, K, dtype)
        x = H.to_device_bits(xb, dtype)
        y0 = w4.gemv(x, pw, workspace=w4.Workspace("cuda"))
        torch.cuda.synchronize()
        H.check_against_oracle(y0, xb, dtype, o, group)
        nbytes = w4.workspace_bytes(M, N, K, group)
        for fill in ("random", "ints"):
            ws = w4.Workspace("cuda")
            buf = ws.get(nbytes)
            if fill == "random":
                buf.copy_(torch.randint(0, 256, buf.shape, dtype=torch.uint8, device="cuda"))
            else:
                words = buf[: buf.numel() // 8 * 8].view(torch.int64)
                words.copy_(torch.arange(words.numel(), dtype=torch.int64, device="cuda") % 7)
            for _ in range(2):
                y = w4.gemv(x, pw, workspace=ws)
                torch.cuda.synchronize()
                assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), fill
        ws = w4.Workspace("cuda")
        out = torch.empty_like(y0)
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            w4.gemv(x, pw, out=out, workspace=ws, stream=stream)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                w4.gemv(x, pw, out=out, workspace=ws, stream=stream)
        for i in range(3):
            out.zero_()
            filler = torch.randn(1 << 18, device="cuda").sum()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), y0.view(torch.int16)), f"replay {i}"
            assert bool(torch.isfinite(filler))
    H.drop(("split", N, K, group))


def test_split_k_decode_short_workspace_refused():
    import torch
    w4 = H.lib()
    N, K, group = 136, 65536, 128
    w, o, pw = H.prepared(("split", N, K, group), lambda: wl.random_weights(N * 7 + K, N, K), group)
    x = H.to_device_bits(wl.random_activations(2, 1, K, "f16"), "f16")
    nbytes = w4.workspace_bytes(1, N, K, group)
    assert nbytes > 0
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.full((1, N), 2.0, dtype=torch.float16, device="cuda")
    args = (x.data_ptr(), 0, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(), y.data_ptr(), 1, N, K, group)
    for fn in ("w4a16_gemv", "w4a16_linear"):
        assert getattr(w4.raw(), fn)(*args, buf.data_ptr(), nbytes - 1, None) == 4, fn   # W4A16_ERR_WORKSPACE
        assert getattr(w4.raw(), fn)(*args, None, 0, None) == 4, fn
    torch.cuda.synchronize()
    assert bool((y == 2.0).all())
