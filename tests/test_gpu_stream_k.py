"""GPU parity of the stream-K schedule of the tiled GEMM: shapes whose tile count
leaves a partly idle last round on the 256 compute units split the last rounds'
tiles by columns over 256 workgroups, which hand fp32 partial tiles over
through the workspace. Outputs within the bar of the oracle (R19), one-hot
inputs bit-exact, repeat calls and graph replays bit-identical, any workspace
contents accepted, a short workspace refused."""
import numpy as np
import pytest

import workloads as wl
from oracle import w4a16_ref as ref
from tests import helpers as H

pytestmark = pytest.mark.gpu

# (M, N, K, group), 256 x 256 tiles: 8 x 33 = 264 tiles (a last round of 8
# tiles: every workgroup shares tiles), the same with ragged K (a partial last
# column in the tail segments), with group 64, with group 256 (one metadata
# slot per two columns) and with ragged M (the last tile row holds 208 rows),
# and 8 x 97 = 776 tiles (two rounds of whole tiles, then the last 264 tiles
# split)
SK_SHAPES = [(2048, 8448, 2048, 128), (2048, 8448, 2080, 32), (2048, 8448, 2048, 64), (2048, 8448, 2048, 256),
             (2000, 8448, 2048, 128), (2048, 24832, 2048, 128)]


def _prep(N, K, group, fmt="asym4"):
    return H.prepared(("sk", N, K, group), lambda: wl.random_weights(N * 3 + K, N, K), group, fmt)


def _cols(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(16), N - 16 + np.arange(16), rng.choice(N, 96, replace=False)]))


def _uses_stream_k(M, N, K, group):
    return H.lib().workspace_bytes(M, N, K, group) > 0


@pytest.mark.parametrize("M,N,K,group", SK_SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_stream_k_matches_oracle(M, N, K, group, dtype):
    import torch
    assert _uses_stream_k(M, N, K, group), "shape expected to take the stream-K split"
    w, o, pw = _prep(N, K, group)
    x = wl.random_activations(M + N + K, M, K, dtype)
    y = H.lib().gemm(H.to_device_bits(x, dtype), pw)
    torch.cuda.synchronize()
    H.check_against_oracle(y, x, dtype, o, group, cols=_cols(N, M + K))
    # every output row of a few columns: each tile's rows, split or whole
    H.check_against_oracle(y, x, dtype, o, group, cols=np.array([0, 255, 256, N // 2, N - 1]))


@pytest.mark.parametrize("fmt", ["sym8", "kq4"])
def test_stream_k_formats(fmt):
    import torch
    M, N, K = 2048, 8448, 2048
    group = 256 if fmt == "kq4" else 128
    w, o, pw = _prep(N, K, group, fmt)
    x = wl.random_activations(7, M, K, "bf16")
    y = H.lib().gemm(H.to_device_bits(x, "bf16"), pw)
    torch.cuda.synchronize()
    H.check_against_oracle(y, x, "bf16", o, group, cols=_cols(N, 3))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_stream_k_one_hot_is_exact(dtype):
    """One-hot rows: one of the two halves of a split tile holds the selected
    weight and the other an exact zero, so the sum is round(w_hat) exactly."""
    import torch
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    w_hat = ref.dequantize(o["codes"], o["s_bits"], o["zeros"], group)
    ks = (np.arange(M) * 7919 + 3) % K
    x32 = np.zeros((M, K), dtype=np.float32)
    x32[np.arange(M), ks] = 1.0
    y = H.lib().gemm(H.to_device_bits(wl.to_16bit(x32, dtype), dtype), pw)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    cols = _cols(N, 11)
    want = ref.out_round_bits(w_hat[cols][:, ks].T, dtype)
    assert np.array_equal(got[:, cols], want)


def test_stream_k_repeatable_any_workspace_and_graph_replay():
    import torch
    w4 = H.lib()
    M, N, K, group = 2048, 8448, 2080, 32
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(5, M, K, "bf16"), "bf16")
    nbytes = w4.workspace_bytes(M, N, K, group)
    # a workspace full of arbitrary bytes (stale flags included) gives the same result
    ws_a, ws_b = w4.Workspace("cuda"), w4.Workspace("cuda")
    buf = ws_b.get(nbytes)
    buf.copy_(torch.randint(0, 256, buf.shape, dtype=torch.uint8, device="cuda"))
    y0 = w4.gemm(x, pw, workspace=ws_a)
    y1 = w4.gemm(x, pw, workspace=ws_b)
    y2 = w4.gemm(x, pw, workspace=ws_a)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))
    # replays of one captured launch (one token): each must wait for its own partials
    out = torch.empty_like(y0)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        w4.gemm(x, pw, out=out, workspace=ws_a)   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            w4.gemm(x, pw, out=out, workspace=ws_a)
    for i in range(3):
        out.zero_()
        filler = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y0.view(torch.int16)), f"replay {i}"
        assert bool(torch.isfinite(filler))


def test_stream_k_workspace_holding_small_integers():
    """A workspace whose every 8-byte word holds a small integer (what ids,
    positions or a launch counter would leave there) gives the result of a
    clean one: the hand-over tokens are 64-bit mixes of a random seed, so no
    stale word passes for a flag."""
    import torch
    w4 = H.lib()
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(9, M, K, "f16"), "f16")
    nbytes = w4.workspace_bytes(M, N, K, group)
    want = w4.gemm(x, pw, workspace=w4.Workspace("cuda"))
    for base in (0, 1, 1 << 20):
        ws = w4.Workspace("cuda")
        buf = ws.get(nbytes)
        words = buf[: buf.numel() // 8 * 8].view(torch.int64)
        words.copy_(torch.arange(base, base + words.numel(), dtype=torch.int64, device="cuda"))
        for _ in range(3):
            y = w4.gemm(x, pw, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want.view(torch.int16)), base


def test_stream_k_wait_expiry_poisons_tiles_and_reports():
    """The testing hook makes every waiting workgroup's bounded wait run out
    (its token is never written): all kernels end, each split tile of y is NaN
    as a whole, every other output equals the normal call, and the next compute
    call, whichever it is, returns W4A16_ERR_HIP once; the one after runs."""
    import torch
    w4 = H.lib()
    raw = w4.raw()
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(8, M, K, "bf16"), "bf16")
    nbytes = w4.workspace_bytes(M, N, K, group)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    want = w4.gemm(x, pw)
    torch.cuda.synchronize()
    y = torch.zeros_like(want)
    head = (x.data_ptr(), 1, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr())
    assert raw.w4a16_testing_gemm_expire(*head, y.data_ptr(), M, N, K, group, 0, ws.data_ptr(), nbytes, None) == 0
    torch.cuda.synchronize()
    nan = torch.isnan(y.float())
    # tiles are 64, 128 or 256 rows by 256 columns: every 64 x 256 block is all NaN or none
    per_block = nan.view(M // 64, 64, N // 256, 256).sum(dim=(1, 3))
    assert bool(((per_block == 0) | (per_block == 64 * 256)).all())
    assert int(per_block.count_nonzero()) > 0
    assert torch.equal(y.view(torch.int16)[~nan], want.view(torch.int16)[~nan])
    # the error is reported by the next call (here an unrelated decode call) and then cleared
    x1 = H.to_device_bits(wl.random_activations(3, 1, K, "bf16"), "bf16")
    y1 = torch.zeros((1, N), dtype=torch.bfloat16, device="cuda")
    st = raw.w4a16_linear(x1.data_ptr(), 1, *head[2:], y1.data_ptr(), 1, N, K, group, None, 0, None)
    assert st == 3, st   # W4A16_ERR_HIP, nothing enqueued
    torch.cuda.synchronize()
    assert not bool(y1.float().abs().sum())
    y2 = torch.zeros_like(want)
    assert raw.w4a16_gemm(*head, y2.data_ptr(), M, N, K, group, ws.data_ptr(), nbytes, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), want.view(torch.int16))


def test_testing_hook_refuses_shapes_without_a_split():
    import torch
    w4 = H.lib()
    M, N, K, group = 256, 8448, 512, 128
    assert w4.workspace_bytes(M, N, K, group) == 0
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(4, M, K, "f16"), "f16")
    y = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    st = w4.raw().w4a16_testing_gemm_expire(x.data_ptr(), 0, pw.qweight.data_ptr(), pw.scales.data_ptr(),
                                            pw.zeros_ptr(), y.data_ptr(), M, N, K, group, 0, None, 0, None)
    assert st == 1   # W4A16_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


def test_default_workspace_is_per_stream():
    """Calls on two streams without an explicit workspace run at the same
    time on workspaces of their own: every result equals the serial one."""
    import threading
    import torch
    w4 = H.lib()
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    xs = [H.to_device_bits(wl.random_activations(300 + i, M, K, "f16"), "f16") for i in range(2)]
    want = [w4.gemm(x, pw) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(4):
                    y = w4.gemm(xs[i], pw)
                    streams[i].synchronize()
                    if not torch.equal(y.view(torch.int16), want[i].view(torch.int16)):
                        errors.append(f"stream {i}: split GEMM differs")
        except Exception as e:   # reported below
            errors.append(f"stream {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    from w4a16_weight_only_dequant_amd import _lib
    keys = {k for k in _lib._workspaces if k[1] in (s.cuda_stream for s in streams)}
    assert len(keys) == 2


def test_stream_k_short_workspace_refused():
    import torch
    w4 = H.lib()
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(6, M, K, "f16"), "f16")
    nbytes = w4.workspace_bytes(M, N, K, group)
    assert nbytes >= 256 * 256 * 256 * 4
    short = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = w4.raw().w4a16_gemm(x.data_ptr(), 0, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(),
                             y.data_ptr(), M, N, K, group, short.data_ptr(), short.numel(), None)
    assert st == 4
    st = w4.raw().w4a16_gemm(x.data_ptr(), 0, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(),
                             y.data_ptr(), M, N, K, group, None, 0, None)
    assert st == 4


def test_stream_k_through_grouped_and_awq_calls():
    """The grouped call (large M: one tiled launch per problem, sharing the
    workspace) and the AWQ path (scaled activations, then the product's own
    workspace after them) on a split shape match w4a16_gemm bit for bit."""
    import torch
    w4 = H.lib()
    M, K, group = 2048, 2048, 128
    pw_a = _prep(8448, K, group)[2]          # splits (264 tiles)
    pw_b = H.prepared(("sk-whole", 4096, K, group), lambda: wl.random_weights(41, 4096, K), group)[2]   # whole tiles
    assert w4.workspace_bytes(M, 8448, K, group) > 0 and w4.workspace_bytes(M, 4096, K, group) == 0
    x = H.to_device_bits(wl.random_activations(13, M, K, "bf16"), "bf16")
    ys = w4.linear_group([x, x], [pw_b, pw_a])    # the problem needing a workspace comes second
    singles = [w4.gemm(x, pw_b), w4.gemm(x, pw_a)]
    torch.cuda.synchronize()
    for y, s in zip(ys, singles):
        assert torch.equal(y.view(torch.int16), s.view(torch.int16))
    m = torch.full((K,), 0.5, dtype=torch.float32, device="cuda")
    y_awq = w4.linear_awq(x, m, pw_a)
    y_pre = w4.gemm(w4.scale_activations(x, m), pw_a)
    torch.cuda.synchronize()
    assert torch.equal(y_awq.view(torch.int16), y_pre.view(torch.int16))


@pytest.mark.parametrize("N,K,split", [(12288, 2048, True), (12544, 2048, False), (16640, 2048, True),
                                       (24832, 2048, True), (36864, 2048, False), (12288, 1920, False)])
def test_stream_k_plan_boundaries(N, K, split):
    """M = 2048 (256-row tiles, 8 per column of tiles) on 256 compute units,
    K = 2048 (16 columns): 384 tiles (last round exactly half full: split),
    392 (just over: whole), 520 (one whole round, then the last two split),
    776 (four rounds, the last of 8 tiles: split) and 1152 (five rounds:
    whole); K = 1920 (15 columns: whole). Outputs within the bar either way."""
    import torch
    M, group = 2048, 128
    assert _uses_stream_k(M, N, K, group) == split
    w, o, pw = _prep(N, K, group)
    x = wl.random_activations(N + 5, M, K, "bf16")
    y = H.lib().linear(H.to_device_bits(x, "bf16"), pw)
    torch.cuda.synchronize()
    H.check_against_oracle(y, x, "bf16", o, group, cols=_cols(N, N))
    H.drop(("sk", N, K, group))


def test_concurrent_calls_on_two_streams():
    """Two host threads, each with its own stream and workspace, run split
    (stream-K) and decode calls at the same time: every result equals the
    serial one (per-launch tokens, per-device attribute records and the
    plan caches are safe to share)."""
    import threading
    import torch
    w4 = H.lib()
    M, N, K, group = 2048, 8448, 2048, 128
    w, o, pw = _prep(N, K, group)
    xs = [H.to_device_bits(wl.random_activations(100 + i, M, K, "bf16"), "bf16") for i in range(2)]
    x1 = [H.to_device_bits(wl.random_activations(200 + i, 1, K, "f16"), "f16") for i in range(2)]
    want = [w4.gemm(x, pw) for x in xs]
    want1 = [w4.linear(x, pw) for x in x1]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            ws = w4.Workspace("cuda")
            with torch.cuda.stream(stream):
                for _ in range(3):
                    y = w4.gemm(xs[i], pw, workspace=ws, stream=stream)
                    y1 = w4.linear(x1[i], pw, workspace=ws, stream=stream)
                    stream.synchronize()
                    if not torch.equal(y.view(torch.int16), want[i].view(torch.int16)):
                        errors.append(f"thread {i}: split GEMM differs")
                    if not torch.equal(y1.view(torch.int16), want1[i].view(torch.int16)):
                        errors.append(f"thread {i}: decode differs")
        except Exception as e:   # reported below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


@pytest.mark.parametrize("M,N,K,group", [(2048, 8448, 2048, 128), (2048, 24832, 2048, 128), (1024, 8448, 2048, 64),
                                         (2048, 4096, 512, 128), (1, 1024, 8192, 128), (8, 5120, 2048, 32)])
def test_workspace_bytes_are_enough_and_nothing_beyond_is_written(M, N, K, group):
    """Every product call succeeds with exactly w4a16_workspace_bytes of
    workspace, writes nothing past it (a guard region after it keeps its
    pattern) and gives the same output as with a generous workspace; the calls
    whose need it is (the decode kernel at M <= 8, the matrix-core GEMM above,
    and w4a16_linear where it routes to them) are refused with one byte less."""
    import torch
    w4 = H.lib()
    w, o, pw = _prep(N, K, group)
    x = H.to_device_bits(wl.random_activations(M + 3, M, K, "bf16"), "bf16")
    nbytes = w4.workspace_bytes(M, N, K, group)
    guard = 1 << 16
    buf = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    big = torch.zeros(nbytes + (1 << 20), dtype=torch.uint8, device="cuda")
    calls = ["w4a16_gemm", "w4a16_linear"] + (["w4a16_gemv"] if M <= 8 else [])
    for fn in calls:
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y_ref = torch.empty_like(y)
        args = (x.data_ptr(), 1, pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr())
        shape = (M, N, K, group)
        st = getattr(w4.raw(), fn)(*args, y.data_ptr(), *shape, buf.data_ptr() if nbytes else None, nbytes, None)
        assert st == 0, (fn, st)
        assert getattr(w4.raw(), fn)(*args, y_ref.data_ptr(), *shape, big.data_ptr(), big.numel(), None) == 0
        torch.cuda.synchronize()
        assert bool((buf[nbytes:] == 0xA5).all()), f"{fn} wrote past its workspace"
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), fn
        needy = ["w4a16_gemv" if M <= 8 else "w4a16_gemm"] + (["w4a16_linear"] if M <= w4.gemv_max_m() or M > 8
                                                               else [])
        if nbytes and fn in needy:
            assert getattr(w4.raw(), fn)(*args, y.data_ptr(), *shape, buf.data_ptr(), nbytes - 1, None) == 4, fn
    H.check_against_oracle(y, wl.random_activations(M + 3, M, K, "bf16"), "bf16", o, group, cols=_cols(N, 5))
    H.drop(("sk", N, K, group))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_stream_k_every_output(dtype):
    """M = 2048, N = 8448, K = 2048: 264 tiles, all split over the 256
    workgroups; every output against the oracle."""
    import torch
    M, N, K, group = 2048, 8448, 2048, 128
    assert _uses_stream_k(M, N, K, group)
    w, o, pw = _prep(N, K, group)
    x = wl.random_activations(78, M, K, dtype)
    y = H.lib().linear(H.to_device_bits(x, dtype), pw)
    torch.cuda.synchronize()
    H.check_every_output(y, x, dtype, o, group)


def test_stream_k_full_size_ffn_shape():
    """M = 2048, N = 11008, K = 4096 (a 7B-style FFN width: 344 tiles, the last
    two rounds split): long segments of 32-column tiles, every row of 160
    sampled columns against the oracle."""
    import torch
    M, N, K, group = 2048, 11008, 4096, 128
    assert _uses_stream_k(M, N, K, group)
    w, o, pw = _prep(N, K, group)
    x = wl.random_activations(77, M, K, "bf16")
    y = H.lib().linear(H.to_device_bits(x, "bf16"), pw)
    torch.cuda.synchronize()
    H.check_against_oracle(y, x, "bf16", o, group, cols=np.unique(np.concatenate([_cols(N, 8), N - 256 + np.arange(32)])))
    H.drop(("sk", N, K, group))
