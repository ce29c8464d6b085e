"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, sizes buffers by the closed form, and rejects bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def w4():
    import w4a16_weight_only_dequant_amd as w4
    return w4


def test_library_exports_every_declared_symbol(w4):
    lib = ctypes.CDLL(w4.LIB_PATH)
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(w4.EXPORTED)


def test_library_exports_only_the_c_abi(w4):
    """The dynamic symbol table holds the declared C entry points and nothing
    else (internal C++ symbols are local to the library)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not installed")
    out = subprocess.run([nm, "-D", "--defined-only", w4.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert exported == set(_declared())


def test_status_strings_and_version(w4):
    lib = w4.raw()
    assert lib.w4a16_layout_version() == 3
    for code in range(5):
        assert lib.w4a16_status_string(code)
    assert lib.w4a16_status_string(99) == b"unknown status"


@pytest.mark.parametrize("N,K,group", [(4096, 4096, 128), (8192, 28672, 32), (5120, 13824, 128), (72, 96, 32),
                                       (72, 192, 64), (72, 160, 32)])
def test_packed_bytes_closed_form(w4, N, K, group):
    G = K // group
    q, s, z = w4.packed_bytes(N, K, group)
    assert q == N * K // 2
    # metadata row-major, each row's G groups padded to a multiple of 8 slots;
    # exactly 2GN / GN/2 when G % 8 == 0
    slots = -(-G // 8) * 8
    assert (s, z) == (2 * slots * N, slots * N // 2)
    if G % 8 == 0:
        assert (s, z) == (2 * G * N, G * N // 2)


@pytest.mark.parametrize("N,K,group", [(100, 128, 128), (4, 128, 128), (64, 100, 32), (64, 128, 16),
                                       (64, 64, 128), (64, 0, 32)])
def test_bad_shapes_rejected(w4, N, K, group):
    with pytest.raises(w4.W4A16Error) as e:
        w4.packed_bytes(N, K, group)
    assert e.value.status == 1


def test_workspace_sizes_monotone_and_bounded(w4):
    for M in (1, 2, 8, 16, 64, 2048):
        b = w4.workspace_bytes(M, 4096, 4096, 128)
        assert 0 <= b <= 64 * M * 4096 * 4 + (1 << 16)


def test_compute_calls_validate_before_device(w4):
    lib = w4.raw()
    ws = ctypes.c_size_t(0)
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation first
    # NULL x
    assert lib.w4a16_gemv(None, 0, fake, fake, fake, fake, 1, 64, 128, 128, None, 0, None) == 1
    # bad dtype
    assert lib.w4a16_gemm(fake, 7, fake, fake, fake, ctypes.c_void_p(1 << 30), 1, 64, 128, 128, None, 0, None) == 1
    # M > 8 on the GEMV entry point
    assert lib.w4a16_gemv(fake, 0, fake, fake, fake, fake, 9, 64, 128, 128, None, 0, None) == 1
    # misaligned pointer
    assert lib.w4a16_linear(ctypes.c_void_p((1 << 20) + 2), 0, fake, fake, fake, ctypes.c_void_p(1 << 30),
                            1, 64, 128, 128, None, 0, None) == 1
    # y overlapping x
    assert lib.w4a16_gemm(fake, 0, ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31), ctypes.c_void_p(1 << 32),
                          fake, 4, 64, 128, 128, None, 0, None) == 1
    # group / shape
    assert lib.w4a16_gemv(fake, 0, fake, fake, fake, fake, 1, 64, 128, 48, None, 0, None) == 1
    assert lib.w4a16_pack(None, 64, 128, 128, fake, fake, fake, None) == 1
    assert lib.w4a16_unpack(fake, fake, fake, 60, 128, 128, fake, fake, fake, None) == 1
    assert lib.w4a16_workspace_bytes(-1, 64, 128, 128, ctypes.byref(ws)) == 1


def test_awq_workspace_must_not_overlap_the_weights(w4):
    """The unfused AWQ path (M > 8) writes the scaled activations into the
    workspace: a workspace that overlaps the packed codes, scales or
    zero-points is refused before the device is touched."""
    lib = w4.raw()
    M, N, K, g = 16, 64, 256, 128
    ws = ctypes.c_size_t(0)
    assert lib.w4a16_awq_workspace_bytes(M, N, K, g, 0, 0, ctypes.byref(ws)) == 0 and ws.value >= M * K * 2
    x, m, q, s, z, y = (ctypes.c_void_p(a << 24) for a in (1, 2, 3, 4, 5, 6))   # never dereferenced
    for at in (q, s, z):
        assert lib.w4a16_linear_awq(x, 0, m, q, s, z, y, M, N, K, g, 0, at, ws.value, None) == 1


def test_empty_batch_is_a_no_op(w4):
    """M = 0: the shape, type and format arguments are checked, no pointer is
    read (all NULL here), nothing is enqueued (no device is needed), OK."""
    lib = w4.raw()
    ws = ctypes.c_size_t(7)
    assert lib.w4a16_workspace_bytes(0, 64, 128, 128, ctypes.byref(ws)) == 0 and ws.value == 0
    for name in ("w4a16_gemv", "w4a16_gemm", "w4a16_linear"):
        fn = getattr(lib, name)
        assert fn(None, 0, None, None, None, None, 0, 64, 128, 128, None, 0, None) == 0, name
        assert fn(None, 1, None, None, None, None, 0, 64, 256, 32, None, 0, None) == 0, name
        assert fn(None, 0, None, None, None, None, 0, 60, 128, 128, None, 0, None) == 1, name   # N % 8
        assert fn(None, 0, None, None, None, None, 0, 64, 128, 48, None, 0, None) == 1, name    # group
        assert fn(None, 7, None, None, None, None, 0, 64, 128, 128, None, 0, None) == 1, name   # dtype
        assert fn(None, 0, None, None, None, None, -1, 64, 128, 128, None, 0, None) == 1, name  # M < 0
        fmt = getattr(lib, name + "_fmt")
        assert fmt(None, 0, None, None, None, None, 0, 64, 256, 256, 3, None, 0, None) == 0, name
        assert fmt(None, 0, None, None, None, None, 0, 64, 256, 128, 3, None, 0, None) == 1, name   # kq4 needs 256
        assert fmt(None, 0, None, None, None, None, 0, 64, 256, 128, 9, None, 0, None) == 1, name   # format
    assert lib.w4a16_linear_awq(None, 0, None, None, None, None, None, 0, 64, 256, 128, 0, None, 0, None) == 0
    assert lib.w4a16_linear_awq(None, 0, None, None, None, None, None, 0, 64, 200, 128, 0, None, 0, None) == 1
    assert lib.w4a16_scale_activations(None, 0, None, None, 0, 64, None) == 0
    assert lib.w4a16_scale_activations(None, 0, None, None, 0, 60, None) == 1
    assert lib.w4a16_awq_workspace_bytes(0, 64, 256, 128, 0, 0, ctypes.byref(ws)) == 0 and ws.value == 0
    Ns = (ctypes.c_int64 * 2)(64, 128)
    assert lib.w4a16_linear_group(2, None, 0, None, None, None, None, 0, Ns, 128, 128, None, 0, None) == 0
    bad = (ctypes.c_int64 * 2)(64, 60)
    assert lib.w4a16_linear_group(2, None, 0, None, None, None, None, 0, bad, 128, 128, None, 0, None) == 1
    assert lib.w4a16_linear_kernel(0, 64, 128, 128, 0) == -1


def test_grouped_call_validates_before_device(w4):
    lib = w4.raw()


    def arr(*v):
        return (ctypes.c_void_p * len(v))(*v)

    a, b, c, d = (1 << 20), (1 << 24), (1 << 28), (1 << 32)
    ok_y = arr(1 << 36, 1 << 37)
    Ns = (ctypes.c_int64 * 2)(64, 64)
    args = lambda count, x, y, N, M=1: (count, x, 0, arr(b, b + (1 << 22)), arr(c, c + (1 << 22)),  # noqa: E731
                                        arr(d, d + (1 << 22)), y, M, N, 128, 128, None, 0, None)
    # count out of range
    assert lib.w4a16_linear_group(*args(0, arr(a, a), ok_y, Ns)) == 1
    assert lib.w4a16_linear_group(*args(9, arr(a, a), ok_y, Ns)) == 1
    # one problem with a bad N
    assert lib.w4a16_linear_group(*args(2, arr(a, a), ok_y, (ctypes.c_int64 * 2)(64, 60))) == 1
    # the output of problem 1 overlapping the activations of problem 0
    assert lib.w4a16_linear_group(*args(2, arr(a, a + (1 << 22)), arr(1 << 36, a), Ns)) == 1
    # NULL arrays
    assert lib.w4a16_linear_group(2, None, 0, None, None, None, None, 1, Ns, 128, 128, None, 0, None) == 1


def test_missing_workspace_reported(w4):
    lib = w4.raw()
    shapes = [(M, N, K, g) for M in (1, 4, 16, 64, 256) for (N, K, g) in
              ((4096, 4096, 128), (8192, 28672, 32), (15360, 5120, 128))]
    needy = [s for s in shapes if w4.workspace_bytes(*s) > 0]
    if not needy:
        pytest.skip("no shape needs a workspace in this build")
    # the decode kernel's split-K workspace (M <= 8) and the tiled GEMM's (large M)
    cases = [("w4a16_gemv", s) for s in needy if s[0] <= 8][:1] + [("w4a16_gemm", s) for s in needy if s[0] > 8][:1]
    assert cases
    a = [ctypes.c_void_p((1 << 34) + i * (1 << 30)) for i in range(5)]
    for fn, (M, N, K, g) in cases:
        need = w4.workspace_bytes(M, N, K, g)
        st = getattr(lib, fn)(a[0], 0, a[1], a[2], a[3], a[4], M, N, K, g, None, 0, None)
        assert st == 4, fn
        st = getattr(lib, fn)(a[0], 0, a[1], a[2], a[3], a[4], M, N, K, g, ctypes.c_void_p(1 << 40), need - 1, None)
        assert st == 4, fn


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "w4a16_weight_only_dequant_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower().replace("oracle/", ""), f
                assert "w4a16_ref" not in text, f


@pytest.mark.parametrize("N,K,group", [(4096, 4096, 128), (72, 768, 256), (5120, 13824, 256), (72, 160, 32)])
def test_packed_bytes_formats(w4, N, K, group):
    slots = -(-(K // group) // 8) * 8
    assert w4.packed_bytes(N, K, group, "asym4") == (N * K // 2, 2 * slots * N, slots * N // 2)
    assert w4.packed_bytes(N, K, group, "sym4") == (N * K // 2, 2 * slots * N, 0)
    assert w4.packed_bytes(N, K, group, "sym8") == (N * K, 2 * slots * N, 0)
    assert w4.packed_bytes(N, K, group) == w4.packed_bytes(N, K, group, "asym4")


def test_format_arguments_validated(w4):
    lib = w4.raw()
    q, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.w4a16_packed_bytes_fmt(64, 256, 128, 3, ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)) == 1
    assert lib.w4a16_packed_bytes_fmt(64, 384, 256, 1, ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)) == 1
    fake = ctypes.c_void_p(1 << 20)
    y = ctypes.c_void_p(1 << 30)
    # unknown format
    assert lib.w4a16_gemm_fmt(fake, 0, fake, fake, fake, y, 1, 64, 256, 128, 3, None, 0, None) == 1
    assert lib.w4a16_pack_fmt(fake, 64, 256, 128, -1, fake, fake, fake, None) == 1
    # the zero-point format needs its zeros; K % 256 for group 256
    assert lib.w4a16_linear_fmt(fake, 0, fake, fake, None, y, 1, 64, 256, 128, 0, None, 0, None) == 1
    assert lib.w4a16_gemv_fmt(fake, 0, fake, fake, None, y, 1, 64, 384, 256, 1, None, 0, None) == 1
    with pytest.raises(ValueError):
        w4.packed_bytes(64, 256, 128, "int3")
