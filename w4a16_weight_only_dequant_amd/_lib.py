"""ctypes binding of libw4a16.so (the gfx950 HIP library).

Argument marshalling only: every step of the linear layer runs in the HIP
kernels behind the C ABI declared in include/w4a16.h. PyTorch supplies device
memory and the current HIP stream. If the shared library is missing this
module raises at import time; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(_HERE, "libw4a16.so")

W4A16_OK = 0
W4A16_F16 = 0
W4A16_BF16 = 1
# weight formats (w4a16_format): 4-bit codes + fp16 scale + 4-bit zero-point per
# group; symmetric 4-bit codes; symmetric 8-bit codes (W8A16); K-quant-style
# 256-weight super-blocks (group 256)
FORMATS = {"asym4": 0, "sym4": 1, "sym8": 2, "kq4": 3}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc, gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_szp = ctypes.POINTER(ctypes.c_size_t)
_vpp = ctypes.POINTER(ctypes.c_void_p)
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "w4a16_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a16_layout_version": (ctypes.c_int, []),
    "w4a16_gemv_max_m": (_i32, []),
    "w4a16_linear_kernel": (_i32, [_i64, _i64, _i64, _i32, _i32]),
    "w4a16_linear_launch_shape": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i64p, ctypes.POINTER(_i32)]),
    "w4a16_device_supported": (ctypes.c_int, [ctypes.c_int]),
    "w4a16_init": (ctypes.c_int, [ctypes.c_int]),
    "w4a16_packed_bytes": (ctypes.c_int, [_i64, _i64, _i32, _szp, _szp, _szp]),
    "w4a16_workspace_bytes": (ctypes.c_int, [_i64, _i64, _i64, _i32, _szp]),
    "w4a16_group_workspace_bytes": (ctypes.c_int, [_i32, _i64, _i64p, _i64, _i32, _i32, _szp]),
    "w4a16_pack": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_unpack": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_gemv": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "w4a16_gemm": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "w4a16_linear": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "w4a16_linear_group": (ctypes.c_int, [_i32, _vpp, _i32, _vpp, _vpp, _vpp, _vpp, _i64, _i64p, _i64, _i32,
                                          _vp, _sz, _vp]),
    "w4a16_packed_bytes_fmt": (ctypes.c_int, [_i64, _i64, _i32, _i32, _szp, _szp, _szp]),
    "w4a16_pack_fmt": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_unpack_fmt": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_gemv_fmt": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]),
    "w4a16_gemm_fmt": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]),
    "w4a16_linear_fmt": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz,
                                        _vp]),
    "w4a16_linear_group_fmt": (ctypes.c_int, [_i32, _vpp, _i32, _vpp, _vpp, _vpp, _vpp, _i64, _i64p, _i64, _i32,
                                              _i32, _vp, _sz, _vp]),
    "w4a16_quant_error_workspace_bytes": (ctypes.c_int, [_i64, _i64, _i32, _szp]),
    "w4a16_quant_error": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "w4a16_scale_activations": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _vp]),
    "w4a16_awq_workspace_bytes": (ctypes.c_int, [_i64, _i64, _i64, _i32, _i32, _i32, _szp]),
    "w4a16_linear_awq": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz,
                                        _vp]),
    "w4a16_kernel_workspace_bytes": (ctypes.c_int, [_i32, _i64, _i64, _i64, _i32, _i32, _szp]),
    "w4a16_linear_run_fmt": (ctypes.c_int, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp,
                                            _sz, _vp]),
    "w4a16_linear_noalloc": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "w4a16_measure_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "w4a16_measure_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "w4a16_testing_gemm_expire": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp,
                                                 _sz, _vp]),
}

EXPORTED = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.w4a16_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def _check(fn: str, status: int):
    if status != W4A16_OK:
        raise W4A16Error(fn, status)


def raw():
    """The ctypes handle, for tests of the C ABI itself."""
    return _lib


def _stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return W4A16_F16
    if t.dtype == torch.bfloat16:
        return W4A16_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _fmt_code(fmt: str) -> int:
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown weight format {fmt!r}; one of {sorted(FORMATS)}") from None


def packed_bytes(N: int, K: int, group: int, fmt: str = "asym4"):
    q, s, z = _sz(), _sz(), _sz()
    _check("w4a16_packed_bytes_fmt", _lib.w4a16_packed_bytes_fmt(N, K, group, _fmt_code(fmt), ctypes.byref(q),
                                                                 ctypes.byref(s), ctypes.byref(z)))
    return q.value, s.value, z.value


def workspace_bytes(M: int, N: int, K: int, group: int) -> int:
    b = _sz()
    _check("w4a16_workspace_bytes", _lib.w4a16_workspace_bytes(M, N, K, group, ctypes.byref(b)))
    return b.value


def init(device: int = 0):
    """One-time set-up of a device (w4a16_init); the compute calls run it on first use."""
    _check("w4a16_init", _lib.w4a16_init(device))


def device_supported(device: int = 0) -> bool:
    st = _lib.w4a16_device_supported(device)
    if st not in (0, 2):
        _check("w4a16_device_supported", st)
    return st == 0


def gemv_max_m() -> int:
    return int(_lib.w4a16_gemv_max_m())


LINEAR_KERNELS = ("gemv", "small_batch", "tiled")


def linear_launch_shape(M: int, N: int, K: int, group: int, dtype=torch.float16, fmt: str = "asym4"):
    """(kernel name, workgroups, threads per workgroup) of w4a16_linear's launch."""
    wg, th = ctypes.c_int64(), _i32()
    code = int(_lib.w4a16_linear_launch_shape(M, N, K, group, W4A16_BF16 if dtype == torch.bfloat16 else W4A16_F16,
                                              _fmt_code(fmt), ctypes.byref(wg), ctypes.byref(th)))
    if code < 0:
        raise ValueError("w4a16_linear rejects this shape")
    return LINEAR_KERNELS[code], wg.value, th.value


def linear_kernel(M: int, N: int, K: int, group: int, dtype=torch.float16) -> str:
    """Name of the kernel w4a16_linear uses for this shape (needs a device)."""
    code = int(_lib.w4a16_linear_kernel(M, N, K, group, W4A16_BF16 if dtype == torch.bfloat16 else W4A16_F16))
    if code < 0:
        raise ValueError("w4a16_linear rejects this shape")
    return LINEAR_KERNELS[code]


class PackedWeight:
    """Packed weight of an N x K linear layer, resident in device memory."""

    def __init__(self, qweight, scales, zeros, N, K, group, fmt="asym4"):
        self.qweight = qweight    # uint8 [N*K/2] (sym8: [N*K], two planes), device layout
        self.scales = scales      # float16, per 128-weight column: [T][N][128/group] (group 256: [G][N]);
        #                           kq4: 16-byte super-block records [K/256][N] (viewed as float16)
        self.zeros = zeros        # int32 zero-point words (asym4), None for the symmetric formats
        self.N, self.K, self.group, self.fmt = N, K, group, fmt
        # the kernels index these buffers by the shape alone: check their sizes once here
        qb, sb, zb = packed_bytes(N, K, group, fmt)
        parts = [("qweight", qweight, qb), ("scales", scales, sb)] + ([("zeros", zeros, zb)] if zb else [])
        for name, t, nb in parts:
            if t is None or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous CUDA tensor")
            if t.numel() * t.element_size() < nb:
                raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the layout needs {nb}")
            if t.device != qweight.device:
                raise ValueError("qweight, scales and zeros must be on one device")

    def nbytes(self) -> int:
        z = 4 * self.zeros.numel() if self.zeros is not None else 0
        return self.qweight.numel() + 2 * self.scales.numel() + z

    def zeros_ptr(self):
        return self.zeros.data_ptr() if self.zeros is not None else None


def pack(w: torch.Tensor, group: int, fmt: str = "asym4", stream=None) -> PackedWeight:
    """Quantise fp32 weights [N][K] (device) and pack them (w4a16_pack_fmt)."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_cuda:
        raise TypeError("w must be a 2-D float32 CUDA tensor [N][K]")
    w = w.contiguous()
    N, K = w.shape
    qb, sb, zb = packed_bytes(N, K, group, fmt)
    dev = w.device
    qweight = torch.empty(qb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb // 2, dtype=torch.float16, device=dev)
    zeros = torch.empty(zb // 4, dtype=torch.int32, device=dev) if zb else None
    _check("w4a16_pack_fmt", _lib.w4a16_pack_fmt(w.data_ptr(), N, K, group, _fmt_code(fmt), qweight.data_ptr(),
                                                 scales.data_ptr(), zeros.data_ptr() if zeros is not None else None,
                                                 _stream_ptr(stream)))
    return PackedWeight(qweight, scales, zeros, N, K, group, fmt)


def unpack(pw: PackedWeight, stream=None):
    """Canonical view (codes u8 [N][K], scale bits int16 [G][N], zeros u8 [G][N];
    the symmetric formats report their fixed zero, 8 or 128)."""
    N, K, group = pw.N, pw.K, pw.group
    G = K // group
    dev = pw.qweight.device
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if pw.fmt == "kq4":   # codes only: the super-block records are already canonical
        _check("w4a16_unpack_fmt", _lib.w4a16_unpack_fmt(pw.qweight.data_ptr(), pw.scales.data_ptr(), None, N, K,
                                                         group, _fmt_code(pw.fmt), codes.data_ptr(), None, None,
                                                         _stream_ptr(stream)))
        return codes, None, None
    s_out = torch.empty((G, N), dtype=torch.int16, device=dev)
    z_out = torch.empty((G, N), dtype=torch.uint8, device=dev)
    _check("w4a16_unpack_fmt", _lib.w4a16_unpack_fmt(pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(),
                                                     N, K, group, _fmt_code(pw.fmt), codes.data_ptr(),
                                                     s_out.data_ptr(), z_out.data_ptr(), _stream_ptr(stream)))
    return codes, s_out, z_out


class Workspace:
    """Device workspace handed to the compute calls.

    The calls take a workspace argument sized by w4a16_workspace_bytes: the
    stream-K split of the tiled GEMM keeps its partial tiles there, and every
    other launch needs none (0 bytes), so no buffer is allocated then. The
    buffer only grows; calls that overlap in time need workspaces of their own.
    A buffer used on a stream other than the one it was allocated on is
    recorded on that stream, so that the caching allocator does not hand its
    memory out again before the work queued there is done.
    """

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else torch.device("cuda")
        self.buf = None
        self._alloc_stream = None

    def get(self, nbytes: int, stream=None):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            # the old buffer (if any) was recorded on every stream that used it
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=self.device)
            self._alloc_stream = torch.cuda.current_stream(self.device)
        if stream is not None and stream != self._alloc_stream:
            self.buf.record_stream(stream)
        return self.buf


_workspaces = {}
_workspaces_lock = threading.Lock()


def _default_workspace(device, stream) -> Workspace:
    """One default workspace per (device, stream): calls on different streams
    may run at the same time and must not share partial tiles and flags."""
    key = (device.index, stream.cuda_stream)
    with _workspaces_lock:
        ws = _workspaces.get(key)
        if ws is None:
            ws = _workspaces[key] = Workspace(device)
    return ws


def _output(out, M: int, N: int, x: torch.Tensor) -> torch.Tensor:
    """`out`, checked to be what the call writes (contiguous [M][N] of x's type
    and device), or a new tensor."""
    if out is None:
        return torch.empty((M, N), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (M, N) or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {x.dtype} tensor [{M}][{N}] on {x.device}")
    return out


def _call(fn_name: str, x: torch.Tensor, pw: PackedWeight, out=None, workspace=None, stream=None):
    if x.dim() != 2 or x.shape[1] != pw.K or not x.is_cuda:
        raise ValueError(f"x must be a CUDA tensor [M][{pw.K}]")
    x = x.contiguous()
    M = x.shape[0]
    y = _output(out, M, pw.N, x)
    nbytes = workspace_bytes(M, pw.N, pw.K, pw.group)
    strm = stream if stream is not None else torch.cuda.current_stream(x.device)
    ws = (workspace or _default_workspace(x.device, strm)).get(nbytes, strm)
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_len = ws.numel() if ws is not None else 0
    fn_name = fn_name + "_fmt"
    fn = getattr(_lib, fn_name)
    _check(fn_name, fn(x.data_ptr(), _dtype_code(x), pw.qweight.data_ptr(), pw.scales.data_ptr(),
                       pw.zeros_ptr(), y.data_ptr(), M, pw.N, pw.K, pw.group, _fmt_code(pw.fmt), ws_ptr, ws_len,
                       _stream_ptr(stream)))
    return y


def gemv(x, pw, out=None, workspace=None, stream=None):
    """Decode GEMV (M <= 8): y = x @ w_hat^T."""
    return _call("w4a16_gemv", x, pw, out, workspace, stream)


def gemm(x, pw, out=None, workspace=None, stream=None):
    """MFMA GEMM (any M): y = x @ w_hat^T."""
    return _call("w4a16_gemm", x, pw, out, workspace, stream)


def linear_group(xs, pws, outs=None, workspace=None, stream=None):
    """Several layers of the same M, K, group, format and type in one launch
    (w4a16_linear_group_fmt).

    xs: list of CUDA tensors [M][K] (entries may be the same tensor); pws: list of
    PackedWeight; returns the list of outputs [M][N_p]."""
    count = len(pws)
    if count != len(xs) or count < 1:
        raise ValueError("need one x per packed weight")
    xs = [x.contiguous() for x in xs]
    M, K, group = xs[0].shape[0], pws[0].K, pws[0].group
    for x, pw in zip(xs, pws):
        if x.dim() != 2 or not x.is_cuda or x.shape != (M, K) or x.dtype != xs[0].dtype:
            raise ValueError("every x must be a CUDA tensor [M][K] of one type")
        if pw.K != K or pw.group != group or pw.fmt != pws[0].fmt:
            raise ValueError("every weight must share K, group and format")
    if outs is not None and len(outs) != count:
        raise ValueError("need one output per packed weight")
    ys = [_output(outs[i] if outs is not None else None, M, pw.N, xs[0]) for i, pw in enumerate(pws)]
    arr = lambda vals: (ctypes.c_void_p * count)(*vals)  # noqa: E731
    nb = _sz()
    ns = (ctypes.c_int64 * count)(*[pw.N for pw in pws])
    _check("w4a16_group_workspace_bytes", _lib.w4a16_group_workspace_bytes(count, M, ns, K, group,
                                                                           _fmt_code(pws[0].fmt), ctypes.byref(nb)))
    nbytes = nb.value
    strm = stream if stream is not None else torch.cuda.current_stream(xs[0].device)
    ws = (workspace or _default_workspace(xs[0].device, strm)).get(nbytes, strm)
    zeros = arr([p.zeros_ptr() for p in pws]) if pws[0].zeros is not None else None
    _check("w4a16_linear_group_fmt", _lib.w4a16_linear_group_fmt(
        count, arr([x.data_ptr() for x in xs]), _dtype_code(xs[0]), arr([p.qweight.data_ptr() for p in pws]),
        arr([p.scales.data_ptr() for p in pws]), zeros,
        arr([y.data_ptr() for y in ys]), M, (ctypes.c_int64 * count)(*[p.N for p in pws]), K, group,
        _fmt_code(pws[0].fmt), ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, _stream_ptr(stream)))
    return ys


def linear_run(kernel: str, x, pw, out=None, workspace=None, stream=None):
    """The named kernel ("gemv", "small_batch" or "tiled") instead of
    w4a16_linear's dispatch (w4a16_linear_run_fmt)."""
    code = LINEAR_KERNELS.index(kernel)
    if x.dim() != 2 or x.shape[1] != pw.K or not x.is_cuda:
        raise ValueError(f"x must be a CUDA tensor [M][{pw.K}]")
    x = x.contiguous()
    M = x.shape[0]
    y = _output(out, M, pw.N, x)
    nb = _sz()
    _check("w4a16_kernel_workspace_bytes", _lib.w4a16_kernel_workspace_bytes(code, M, pw.N, pw.K, pw.group,
                                                                             _fmt_code(pw.fmt), ctypes.byref(nb)))
    strm = stream if stream is not None else torch.cuda.current_stream(x.device)
    ws = (workspace or _default_workspace(x.device, strm)).get(nb.value, strm)
    _check("w4a16_linear_run_fmt", _lib.w4a16_linear_run_fmt(
        code, x.data_ptr(), _dtype_code(x), pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(),
        y.data_ptr(), M, pw.N, pw.K, pw.group, _fmt_code(pw.fmt), ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream_ptr(stream)))
    return y


def linear_noalloc(x, pw, out, stream=None):
    """w4a16_linear with the library's static scratch for its workspace: the
    call allocates nothing (out is required; w4a16_init must have run on the
    device). Calls that overlap in time on one device must not be made."""
    if x.dim() != 2 or x.shape[1] != pw.K or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous CUDA tensor [M][{pw.K}]")
    if out is None:
        raise ValueError("linear_noalloc writes into a given out tensor")
    y = _output(out, x.shape[0], pw.N, x)
    _check("w4a16_linear_noalloc", _lib.w4a16_linear_noalloc(
        x.data_ptr(), _dtype_code(x), pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(), y.data_ptr(),
        x.shape[0], pw.N, pw.K, pw.group, _fmt_code(pw.fmt), _stream_ptr(stream)))
    return y


def linear(x, pw, out=None, workspace=None, stream=None):
    """Default path, dispatching on M."""
    return _call("w4a16_linear", x, pw, out, workspace, stream)


QUALITY_FIELDS = ("mse", "snr_db", "cos", "max_err", "sum_d2", "sum_w2", "sum_h2", "sum_wh")


def quant_error(w: torch.Tensor, pw: PackedWeight, stream=None, out=None, workspace=None):
    """Quality report of packed weights against the fp32 weights [N][K] (device)
    they were made from (w4a16_quant_error): MSE, SNR dB, cosine, max error and
    the fp64 sums behind them, as a dict. With `out` (a float64 CUDA tensor of
    8) the report is written there in QUALITY_FIELDS order and `out` is
    returned without waiting for it; `workspace` is a Workspace to reuse."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_cuda or tuple(w.shape) != (pw.N, pw.K):
        raise TypeError(f"w must be a float32 CUDA tensor [{pw.N}][{pw.K}]")
    w = w.contiguous()
    nb = _sz()
    _check("w4a16_quant_error_workspace_bytes",
           _lib.w4a16_quant_error_workspace_bytes(pw.N, pw.K, pw.group, ctypes.byref(nb)))
    ws = (workspace or Workspace(w.device)).get(max(nb.value, 16))
    res = out
    if res is None:
        res = torch.empty(8, dtype=torch.float64, device=w.device)
    elif res.dtype != torch.float64 or res.numel() != 8 or not res.is_contiguous() or res.device != w.device:
        raise ValueError("out must be a contiguous float64 tensor of 8 on the weights' device")
    _check("w4a16_quant_error", _lib.w4a16_quant_error(
        w.data_ptr(), pw.qweight.data_ptr(), pw.scales.data_ptr(), pw.zeros_ptr(), pw.N, pw.K, pw.group,
        _fmt_code(pw.fmt), res.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    if out is not None:
        return out
    return dict(zip(QUALITY_FIELDS, res.cpu().tolist()))


def scale_activations(x: torch.Tensor, act_mul: torch.Tensor, out=None, stream=None):
    """x * act_mul along K, rounded once to x's type (w4a16_scale_activations)."""
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a CUDA tensor [M][K]")
    x = x.contiguous()
    M, K = x.shape
    if act_mul.dtype != torch.float32 or act_mul.numel() != K or not act_mul.is_cuda:
        raise TypeError(f"act_mul must be a float32 CUDA tensor [{K}]")
    y = _output(out, M, K, x)
    _check("w4a16_scale_activations", _lib.w4a16_scale_activations(
        x.data_ptr(), _dtype_code(x), act_mul.contiguous().data_ptr(), y.data_ptr(), M, K, _stream_ptr(stream)))
    return y


def linear_awq(x: torch.Tensor, act_mul: torch.Tensor, pw: PackedWeight, out=None, workspace=None, stream=None):
    """AWQ run-time path: y = (x * act_mul) @ w_hat^T (w4a16_linear_awq); the
    weights are the quantised w * (1 / act_mul)."""
    if x.dim() != 2 or x.shape[1] != pw.K or not x.is_cuda:
        raise ValueError(f"x must be a CUDA tensor [M][{pw.K}]")
    if act_mul.dtype != torch.float32 or act_mul.numel() != pw.K or not act_mul.is_cuda:
        raise TypeError(f"act_mul must be a float32 CUDA tensor [{pw.K}]")
    x = x.contiguous()
    act_mul = act_mul.contiguous()
    M = x.shape[0]
    y = _output(out, M, pw.N, x)
    nb = _sz()
    _check("w4a16_awq_workspace_bytes", _lib.w4a16_awq_workspace_bytes(M, pw.N, pw.K, pw.group, _fmt_code(pw.fmt),
                                                                       _dtype_code(x), ctypes.byref(nb)))
    strm = stream if stream is not None else torch.cuda.current_stream(x.device)
    ws = (workspace or _default_workspace(x.device, strm)).get(nb.value, strm)
    _check("w4a16_linear_awq", _lib.w4a16_linear_awq(
        x.data_ptr(), _dtype_code(x), act_mul.data_ptr(), pw.qweight.data_ptr(), pw.scales.data_ptr(),
        pw.zeros_ptr(), y.data_ptr(), M, pw.N, pw.K, pw.group, _fmt_code(pw.fmt),
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, _stream_ptr(stream)))
    return y
