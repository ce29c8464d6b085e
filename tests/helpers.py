"""Shared helpers for the GPU parity tests: seeded inputs -> oracle -> HIP path."""
from __future__ import annotations

import numpy as np

from oracle import w4a16_ref as ref

_CACHE = {}


def lib():
    import w4a16_weight_only_dequant_amd as w4
    return w4


def oracle_pack(w: np.ndarray, group: int, fmt: str = "asym4"):
    if fmt == "kq4":
        codes, d_bits, m_bits, sc, mq = ref.quantize_kquant(w)
        return {"codes": codes, "fmt": fmt, "kq": (d_bits, m_bits, sc, mq),
                "qweight": ref.pack_device(codes),
                "records": ref.pack_kquant_device(d_bits, m_bits, sc, mq).ravel(),
                "zeros_dev": None}
    codes, s_bits, zeros = ref.quantize_groupwise(w, group, fmt)
    return {
        "codes": codes,
        "s_bits": s_bits,
        "zeros": zeros,
        "fmt": fmt,
        "qweight": ref.pack_device(codes, fmt),
        "scales_dev": ref.pack_scales_device(s_bits, group).ravel(),
        "zeros_dev": ref.pack_zeros_device(zeros, group).ravel() if fmt == "asym4" else None,
    }


def gpu_pack(w: np.ndarray, group: int, fmt: str = "asym4"):
    import torch
    wt = torch.from_numpy(w).cuda()
    pw = lib().pack(wt, group, fmt)
    torch.cuda.synchronize()
    del wt
    return pw


def prepared(key, make_w, group, fmt: str = "asym4"):
    """Weights, oracle quantisation and the GPU-packed weight, cached per key."""
    key = (key, fmt) if fmt != "asym4" else key
    if key not in _CACHE:
        w = make_w()
        o = oracle_pack(w, group, fmt)
        pw = gpu_pack(w, group, fmt)
        _CACHE[key] = (w, o, pw)
    return _CACHE[key]


def drop(key):
    _CACHE.pop(key, None)


def to_device_bits(x_bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def y_to_f64(y) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def check_against_oracle(y_gpu, x_bits, dtype, o, group, cols=None, quiet=False):
    """Assert |y - y_ref| <= 2e-3 * sum|x w_hat| + 1e-5 (bf16 outputs: plus
    half a bf16 ulp, the one rounding to the output type) element-wise; print
    the max ratio to that bar and to the bare bar, return the former."""
    y = y_to_f64(y_gpu)
    if cols is not None:
        y = y[:, cols]
    if o.get("fmt") == "kq4":
        d_bits, m_bits, sc, mq = o["kq"]
        codes = o["codes"]
        if cols is not None:
            codes, d_bits, m_bits = codes[cols], d_bits[:, cols], m_bits[:, cols]
            sc, mq = sc[:, :, cols], mq[:, :, cols]
        y_ref, a = ref.linear_ref(x_bits, dtype, ref.dequantize_kquant(codes, d_bits, m_bits, sc, mq))
    else:
        y_ref, a = ref.linear_ref_rows(x_bits, dtype, o["codes"], o["s_bits"], o["zeros"], group, cols)
    r = ref.error_ratio(y, y_ref, a, dtype)
    worst = float(r.max()) if r.size else 0.0
    bare = float(ref.error_ratio(y, y_ref, a).max()) if r.size else 0.0
    if not quiet:
        print(f"[parity] {y.shape[0]}x{y.shape[1]} outputs: max ratio {worst:.4f} (bare bar {bare:.4f})", flush=True)
    assert np.all(np.isfinite(y)), "non-finite output"
    assert worst <= 1.0, f"max error ratio {worst:.3g} (> 1) at {np.unravel_index(np.argmax(r), r.shape)}"
    return worst


def check_every_output(y_gpu, x_bits, dtype, o, group, chunk=2048):
    """check_against_oracle over every output column, in chunks of columns
    (the fp64 product of a full prefill shape is ~1.5e11 MACs)."""
    N = int(y_gpu.shape[1])
    worst = bare = 0.0
    if o.get("fmt") == "kq4":   # (super-block records: the sliced oracle of check_against_oracle)
        for c0 in range(0, N, chunk):
            cols = np.arange(c0, min(N, c0 + chunk))
            worst = max(worst, check_against_oracle(y_gpu, x_bits, dtype, o, group, cols=cols, quiet=True))
        print(f"[parity] every output of {tuple(y_gpu.shape)}: max ratio {worst:.4f}", flush=True)
        return worst
    for c0 in range(0, N, chunk):
        cols = np.arange(c0, min(N, c0 + chunk))
        y = y_to_f64(y_gpu[:, c0:c0 + len(cols)])
        y_ref, a = ref.linear_ref_rows(x_bits, dtype, o["codes"], o["s_bits"], o["zeros"], group, cols)
        r = ref.error_ratio(y, y_ref, a, dtype)
        assert np.all(np.isfinite(y)), f"non-finite output in columns {c0}.."
        assert float(r.max()) <= 1.0, f"max error ratio {float(r.max()):.3g} (> 1) in columns {c0}.."
        worst = max(worst, float(r.max()))
        bare = max(bare, float(ref.error_ratio(y, y_ref, a).max()))
    print(f"[parity] every output of {tuple(y_gpu.shape)}: max ratio {worst:.4f} (bare bar {bare:.4f})", flush=True)
    return worst
