#!/usr/bin/env python3
"""Benchmark of the gfx950 W4A16 linear layer.

Headline (`value`): the decode layer set of a 13B-class model at M = 1 --
q, k, v, o (K = N = 5120), up and gate (K = 5120, N = 13824), down
(K = 13824, N = 5120), group 128, fp16 activations. One step = one token
through all seven layers (seven w4a16_linear calls, each dispatched to the
decode kernel). `value` is achieved HBM GB/s of the step: algorithmic bytes
(packed weights + scales + zeros + activations read + outputs written) over
wall time per step, K steps replayed from HIP graphs after W warm-up steps.

Legs (`legs`), one per workload, each with its matrices and batch sizes:
  c1 gemv_4096 (M = 1), c2 decode_13b_layer (M = 1, the headline),
  c3 fused_qkv (M = 2, 4, 8, 16), c4 prefill (M = 2048, bf16),
  c5 ffn_down_70b (M = 1, 8; group 32).
Every matrix is timed over a fixed number of launches (--launches, >= 200,
rotated over enough copies of the packed weights to defeat the 256 MB
last-level cache) after a time-based warm-up (50 ms), with HIP events on the
replay stream; the per-launch time includes the dispatch gap between two
dependent launches. Each entry reports the kernel, its launch geometry
(the key of its rows in a rocprofv3 kernel trace), microseconds per launch,
GB/s and TFLOP/s against the HBM and bf16 MFMA peaks, tokens/s, and -- from the
oracle leg -- the bare-bar max error ratio and whether the codes are
bit-exact on the sampled rows.

`roofline`: the dominant kernel of the headline step (the decode kernel): its
algorithmic bytes over its launches' time. `traffic` is filled from committed
counter summaries (profiles/traffic_*.json) when they were taken on the same
kernel sources, else null. `stream_ceiling`: a plain 16-byte streaming read
(w4a16_measure_stream_read) over 2 GiB, and over each decode matrix's bytes at
the decode kernel's grid: the achievable rates, reported beside the kernels.

Other legs: `grouped_step` (q/k/v and up/gate each in one launch,
w4a16_linear_group), `formats` (the decode step and the prefill GEMM with the
weights in the other formats), `quality` (w4a16_quant_error per matrix) and
`awq_step` (the decode step through w4a16_linear_awq).

`cpu_baseline`: the CPU oracle as it stands, timed on the host on sampled rows
of every workload (quantise + pack, then dequantise + fp64 product,
separately), plus a one-thread pass of c1; it also checks the GPU's codes and
outputs on those rows (the legs' max_err_ratio and codes_bitexact).

Profiling modes (for the committed summaries under profiles/):
  --counter-pass DIR  each matrix of each leg launched a few times, eagerly, in
                      a fixed order recorded in DIR/counter_pass.json (the
                      program of a rocprofv3 --pmc run), after a 256 MiB copy
                      kernel that scales the HBM byte counters
  --summarize-trace DIR / --summarize-counters DIR...: read rocprofv3 CSV
                      output and print the summaries (no GPU).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA
MALL_BYTES = 256 << 20
WORKLOAD_IDS = {"gemv_4096": 1, "decode_13b_layer": 2, "fused_qkv": 3, "prefill": 4, "ffn_down_70b": 5}
HEADLINE = 2
WARM_MS = 50.0
CALIBRATION_BYTES = 256 << 20
KERNEL_NAMES = {"gemv": "decode_kernel", "small_batch": "skinny_kernel", "tiled": "prefill_kernel"}
KERNEL_KIND = {"gemv": "gemv", "small_batch": "skinny", "tiled": "prefill"}

# sources each kernel is built from (for matching stored counter results)
KERNEL_SOURCES = {
    "gemv": ["decode.hip", "decode_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
    "skinny": ["gemm.hip", "gemm_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
    "prefill": ["prefill.hip", "prefill_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
}
# weight-format variants measured beside the headline (format, group)
FORMAT_LEGS = [("sym4", 128), ("sym8", 128), ("asym4", 256), ("kq4", 256)]
# rows (output columns) of each matrix the oracle leg works on
ORACLE_ROWS = {1: 4096, 2: 5120, 3: 15360, 4: 13824, 5: 8192}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000, help="timed steps of the headline decode layer set")
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--launches", type=int, default=240, help="timed launches per matrix (>= 200)")
    p.add_argument("--legs", default="1,2,3,4,5", help="workload ids of the legs (2 always runs)")
    p.add_argument("--workload", default=None, choices=list(WORKLOAD_IDS),
                   help="only this workload's leg (with --m: at that M), e.g. for a batch sweep")
    p.add_argument("--m", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-formats", action="store_true", help="skip the weight-format, quality and AWQ legs")
    p.add_argument("--counter-pass", metavar="DIR", default=None)
    p.add_argument("--reps", type=int, default=6, help="launches per matrix in --counter-pass")
    p.add_argument("--summarize-trace", metavar="DIR", default=None)
    p.add_argument("--summarize-counters", metavar="DIR", nargs="+", default=None)
    p.add_argument("--bench-json", default=None, help="a bench.py output line (launch keys of the legs)")
    p.add_argument("--stream-grid", action="store_true",
                   help="time a plain streaming read of each M = 1 decode matrix's bytes at several grids")
    p.add_argument("--crossover", action="store_true",
                   help="time every kernel at M = 1..2048 on two shapes and check the dispatch's choice")
    return p.parse_args()


def kernel_source_hash(kind):
    """Hash of the code a kernel is built from, with comments and all white
    space removed (edits of comments or layout keep stored counters valid)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "w4a16_weight_only_dequant_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        lines = [re.sub(r"\s+", "", re.sub(r"//.*", "", line)) for line in text.splitlines()]
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def decode_variant(kernel, M, N, K, fmt, wgs, threads):
    """The decode kernel's variant a launch runs, from its geometry: one
    activation row, 4-bit codes with a scale per group, whole 128-weight
    columns, one workgroup per row block and sixteen columns per wave (more
    than eight per wave: waves * 8 < columns) run decode_bcast_kernel (the
    library's decode plan), otherwise decode_kernel."""
    cols = K // 128
    if (kernel == "decode_kernel" and M == 1 and fmt in ("asym4", "sym4") and K % 128 == 0
            and wgs == -(-N // 16) and (threads // 64) * 8 < cols):
        return "decode_bcast_kernel"
    return kernel


def algorithmic_bytes(M, N, K, group, fmt="asym4"):
    """Codes (4 or 8 bits per weight), fp16 scales, 4-bit zero-points (asym4
    only), activations read and outputs written."""
    G = K // group
    codes = N * K if fmt == "sym8" else N * K // 2
    zeros = G * N // 2 if fmt == "asym4" else 0
    meta = 16 * (K // 256) * N if fmt == "kq4" else 2 * G * N    # kq4: 16-byte super-block records
    return codes + meta + zeros + 2 * M * K + 2 * M * N


def stored_traffic(workload, M, kind):
    """HBM bytes per launch set from committed counter summaries, if taken on these sources."""
    tfile = os.path.join(ROOT, "profiles", f"traffic_{workload}_m{M}.json")
    if not os.path.exists(tfile):
        return None
    t = json.load(open(tfile))
    if t.get("kernel_source_sha") != kernel_source_hash(kind):
        return None
    return t.get("traffic_bytes_per_launch_set")


def sampled_rows(cfg_id, N):
    """Rows of a matrix the oracle leg checks: whole 16-row blocks (the
    packing unit), the first and the last and a seeded spread, ORACLE_ROWS
    rows in all (every row when that covers N)."""
    import numpy as np
    R = ORACLE_ROWS[cfg_id]
    if R >= N:
        return np.arange(N)
    nb = N // 16
    rng = np.random.default_rng([cfg_id, 77])
    blocks = np.concatenate([[0, nb - 1], 1 + rng.choice(nb - 2, R // 16 - 2, replace=False)])
    return (np.sort(blocks)[:, None] * 16 + np.arange(16)[None, :]).ravel()


_WEIGHTS = {}


def host_weights(cfg_id, j):
    """fp32 weights of one matrix, generated once per process (the oracle leg reuses them)."""
    import workloads as wl
    if (cfg_id, j) not in _WEIGHTS:
        _WEIGHTS[(cfg_id, j)] = wl.weights(cfg_id, j)
    return _WEIGHTS[(cfg_id, j)]


class Workload:
    """Packed weights, activations and outputs of one configuration, with
    enough rotated copies of the weights to defeat the 256 MB MALL."""

    def __init__(self, cfg_id, M, dev, fmt="asym4", group=None):
        import numpy as np
        import torch

        import w4a16_weight_only_dequant_amd as w4
        import workloads as wl
        self.w4, self.torch, self.dev = w4, torch, dev
        self.cfg_id = cfg_id
        self.cfg = wl.WORKLOADS[cfg_id]
        self.M, self.group, self.dtype = M, group or self.cfg.group, self.cfg.dtype
        self.fmt = fmt
        self.tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        self.mats = list(self.cfg.matrices)
        packed, self.xs, self.ys, self.x_bits = [], [], [], []
        for mi, mat in enumerate(self.mats):
            w = torch.from_numpy(host_weights(cfg_id, mi)).to(dev)
            packed.append(w4.pack(w, self.group, fmt))
            del w
            xb = wl.activations(cfg_id, mi, M)
            self.x_bits.append(xb)
            self.xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(self.tdt))
            self.ys.append(torch.empty((M, mat.N), dtype=self.tdt, device=dev))
        torch.cuda.synchronize()
        set_bytes = sum(p.nbytes() for p in packed)
        self.copies = max(1, -(-3 * MALL_BYTES // set_bytes))
        self.sets = [packed]
        for _ in range(self.copies - 1):
            self.sets.append([w4.PackedWeight(p.qweight.clone(), p.scales.clone(),
                                              p.zeros.clone() if p.zeros is not None else None, p.N, p.K,
                                              p.group, p.fmt) for p in packed])
        self.ws = w4.Workspace(dev)
        self.bytes = [algorithmic_bytes(M, m.N, m.K, self.group, fmt) for m in self.mats]
        self.flops = [2 * M * m.N * m.K for m in self.mats]
        self.launch_keys = []
        for m in self.mats:
            kname, wg, th = w4.linear_launch_shape(M, m.N, m.K, self.group, self.tdt, fmt)
            self.launch_keys.append({"kernel": decode_variant(KERNEL_NAMES[kname], M, m.N, m.K, fmt, wg, th),
                                     "kind": KERNEL_KIND[kname], "workgroups": wg, "threads": th})

    def launch(self, c, j):
        self.w4.linear(self.xs[j], self.sets[c][j], out=self.ys[j], workspace=self.ws)

    def step(self, c):
        for j in range(len(self.mats)):
            self.launch(c, j)

    def step_grouped(self, c, groups):
        """One step with the layers of each group in one launch."""
        for g in groups:
            if len(g) == 1:
                self.launch(c, g[0])
            else:
                self.w4.linear_group([self.xs[j] for j in g], [self.sets[c][j] for j in g],
                                     outs=[self.ys[j] for j in g], workspace=self.ws)

    def step_awq(self, c, act_mul):
        """One step through w4a16_linear_awq (activation multipliers per matrix)."""
        for j in range(len(self.mats)):
            self.w4.linear_awq(self.xs[j], act_mul[j], self.sets[c][j], out=self.ys[j], workspace=self.ws)

    def _graph(self, fn):
        torch = self.torch
        cap = torch.cuda.Stream(device=self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn()
        return g

    def time_fn(self, fn, steps, warmup):
        """Wall time per step of fn(copy) replayed from one HIP graph per weight copy."""
        torch = self.torch
        for c in range(min(2, self.copies)):
            fn(c)
        torch.cuda.synchronize()
        graphs = [self._graph(lambda c=c: fn(c)) for c in range(self.copies)]
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % self.copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % self.copies].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def kernel_us(self, j, launches):
        """Microseconds per launch of matrix j: one graph of `launches` launches
        rotating over the weight copies, replayed after a time-based warm-up
        (the device's clocks take milliseconds to rise under a new load);
        HIP events on the replay stream around the timed replay."""
        torch = self.torch
        self.launch(0, j)
        torch.cuda.synchronize()
        n = max(launches, self.copies)
        g = self._graph(lambda: [self.launch(i % self.copies, j) for i in range(n)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < WARM_MS:
            g.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def results_for_oracle(self, rows_of):
        """GPU outputs and unpacked codes on the oracle's sampled rows (copy 0)."""
        torch = self.torch
        out = []
        for j, m in enumerate(self.mats):
            self.launch(0, j)
            rows = rows_of(m.N)
            codes, s, z = self.w4.unpack(self.sets[0][j])
            ridx = torch.from_numpy(rows).to(self.dev)
            out.append({"rows": rows, "y": self.ys[j][:, ridx].float().cpu().numpy().astype("float64"),
                        "codes": codes[ridx].cpu().numpy(), "s_bits": s[:, ridx].cpu().numpy().view("uint16"),
                        "zeros": z[:, ridx].cpu().numpy()})
            del codes, s, z
        torch.cuda.synchronize()
        return out


def rates(nbytes, flops, us, M):
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 3), "GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "TFLOPs": round(tf, 2), "pct_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2),
            "tokens_per_s": round(M / (us * 1e-6), 1)}


def leg_entries(wk, launches):
    entries = {}
    for j, m in enumerate(wk.mats):
        us = wk.kernel_us(j, launches)
        e = {"M": wk.M, "N": m.N, "K": m.K, "bytes_algorithmic": wk.bytes[j], "flops": wk.flops[j],
             "launches": max(launches, wk.copies), "weight_copies": wk.copies, **wk.launch_keys[j]}
        e.update(rates(wk.bytes[j], wk.flops[j], us, wk.M))
        e["roofline_bound"] = "mfma" if e["kind"] == "prefill" else "hbm"
        entries[m.name] = e
    return entries


def run_leg(cfg_id, Ms, dev, launches, stash):
    """One workload: every matrix at every batch size, timed per launch."""
    import torch

    import workloads as wl
    cfg = wl.WORKLOADS[cfg_id]
    leg = {"workload": cfg.name, "group": cfg.group, "dtype": cfg.dtype,
           "seeds": f"numpy default_rng([{cfg_id}, matrix, 0]) weights, ([{cfg_id}, matrix, 1, M]) activations",
           "by_M": {}}
    for M in Ms:
        wk = Workload(cfg_id, M, dev)
        entries = leg_entries(wk, launches)
        if stash is not None:
            stash[(cfg_id, M)] = {"results": wk.results_for_oracle(lambda N: sampled_rows(cfg_id, N)),
                                  "x_bits": wk.x_bits, "entries": entries}
        leg["by_M"][str(M)] = entries
        del wk
        torch.cuda.empty_cache()
    return leg


def headline(dev, steps, warmup, launches, stash):
    """The decode layer set: the timed step, per-kernel times, grouped step."""
    import torch
    M = 1
    wk = Workload(HEADLINE, M, dev)
    for c in range(min(2, wk.copies)):
        wk.step(c)
    torch.cuda.synchronize()
    graphs = [wk._graph(lambda c=c: wk.step(c)) for c in range(wk.copies)]
    for i in range(warmup):
        graphs[i % wk.copies].replay()
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` steps, bracketed by synchronisation ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % wk.copies].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step = {"ms_per_step": wall * 1e3 / steps, "gpu_ms_per_step": e0.elapsed_time(e1) / steps,
            "bytes": sum(wk.bytes), "flops": sum(wk.flops)}
    entries = leg_entries(wk, launches)
    idx = {m.name: j for j, m in enumerate(wk.mats)}
    groups = [[idx[n] for n in g] for g in (("q", "k", "v"), ("o",), ("up", "gate"), ("down",))]
    g_ms = wk.time_fn(lambda c: wk.step_grouped(c, groups), max(200, steps // 2), warmup)
    g_gbs = step["bytes"] / (g_ms * 1e-3) / 1e9
    grouped = {"ms_per_step": round(g_ms, 5), "value": round(g_gbs, 1), "unit": "GB/s",
               "pct_hbm_peak": round(g_gbs / HBM_PEAK_GBS * 100, 2), "launches_per_step": len(groups),
               "groups": [[wk.mats[j].name for j in g] for g in groups], "tokens_per_s": round(M / (g_ms * 1e-3), 1)}
    if stash is not None:
        stash[(HEADLINE, M)] = {"results": wk.results_for_oracle(lambda N: sampled_rows(HEADLINE, N)),
                                "x_bits": wk.x_bits, "entries": entries}
    del wk, graphs
    torch.cuda.empty_cache()
    return step, entries, grouped


def _stream_reader(dev):
    """A 2 GiB device buffer and timed(ptr_fn, nbytes, wgs, reps): microseconds
    per launch of the plain 16-byte streaming read (w4a16_measure_stream_read)
    of nbytes at ptr_fn(i) with wgs workgroups (0: 16 KiB each)."""
    import torch

    import w4a16_weight_only_dequant_amd as w4
    raw = w4.raw()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    big = torch.ones(2 << 30, dtype=torch.uint8, device=dev)

    def timed(ptr_fn, nbytes, wgs, reps):
        """Microseconds per launch: one graph of `reps` launches, replayed
        after a 50 ms warm-up, HIP events around the timed replay."""
        st = raw.w4a16_measure_stream_read(ptr_fn(0), nbytes, sink.data_ptr(), wgs, None)
        assert st == 0, st
        torch.cuda.synchronize()
        cap = torch.cuda.Stream(device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(reps):
                    raw.w4a16_measure_stream_read(ptr_fn(i), nbytes, sink.data_ptr(), wgs, cap.cuda_stream)
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < WARM_MS:
            g.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    return timed, big


def _rotated(big, nbytes):
    """(bytes rounded to 4 KiB, ptr_fn): launch i reads copy i % copies of the
    buffer, with copies x bytes past three times the MALL where the buffer
    holds that many."""
    nb = (nbytes + 4095) // 4096 * 4096
    copies = max(1, min(big.numel() // nb, -(-3 * MALL_BYTES // nb)))
    return nb, (lambda i: big.data_ptr() + (i % copies) * nb)


def stream_ceiling(dev, decode_entries):
    """A plain 16-byte streaming read: over 2 GiB at eight workgroups per
    compute unit, and over each decode matrix's bytes (rotated over copies past
    the MALL) at the decode kernel's number of workgroups."""
    import torch
    timed, big = _stream_reader(dev)
    out = {"kernel": "stream_read_kernel (w4a16_measure_stream_read)"}
    us = timed(lambda i: big.data_ptr(), big.numel(), 0, 20)
    out["2GiB"] = {"bytes": big.numel(), "us": round(us, 1), "GBps": round(big.numel() / us / 1e3, 1),
                   "pct_hbm_peak": round(big.numel() / us / 1e3 / HBM_PEAK_GBS * 100, 2)}
    seen = set()
    for name, e in decode_entries.items():
        key = (e["bytes_algorithmic"], e["workgroups"])
        if key in seen:
            continue
        seen.add(key)
        nb, ptr_fn = _rotated(big, e["bytes_algorithmic"])
        us = timed(ptr_fn, nb, e["workgroups"], 240)
        out[name] = {"bytes": nb, "workgroups": e["workgroups"], "us": round(us, 3),
                     "GBps": round(nb / us / 1e3, 1), "pct_hbm_peak": round(nb / us / 1e3 / HBM_PEAK_GBS * 100, 2),
                     "decode_us": e["us"], "read_over_decode": round(us / e["us"], 3),
                     "note": "the same bytes at the decode launch's number of workgroups, launches replayed "
                             "from a graph like the kernel's"}
    del big
    torch.cuda.empty_cache()
    return out


def stream_grid(dev):
    """The plain streaming read of each M = 1 decode matrix's algorithmic
    bytes at 256 ... 8192 workgroups and at 16 KiB per workgroup (0): how much
    the number of workgroups alone moves the rate a read of that size reaches,
    beside the decode kernel's own grid (profiles/stream_read_vs_grid.txt)."""
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl
    timed, big = _stream_reader(dev)
    cases = [("c1 w", 1, 0), ("c2 q", 2, 0), ("c2 up", 2, 4), ("c2 down", 2, 6), ("c5 down", 5, 0)]
    rows = []
    for label, cfg, mat in cases:
        wlc = wl.WORKLOADS[cfg]
        m = wlc.matrices[mat]
        nbytes = algorithmic_bytes(1, m.N, m.K, wlc.group)
        nb, ptr_fn = _rotated(big, nbytes)
        kern, dec_wgs, _ = w4.linear_launch_shape(1, m.N, m.K, wlc.group, torch.float16)
        for wgs in (256, 320, 512, 864, 1024, 2048, 4096, 8192, 0):
            us = timed(ptr_fn, nb, wgs, 240)
            rows.append({"case": label, "N": m.N, "K": m.K, "group": wlc.group, "bytes": nbytes, "workgroups": wgs,
                         "decode_workgroups": dec_wgs, "us": round(us, 3), "TBps": round(nbytes / us / 1e6, 3)})
            print(f"{label} {wgs} workgroups: {us:.2f} us", file=sys.stderr, flush=True)
    del big
    torch.cuda.empty_cache()
    return rows


def quality_and_awq(dev, steps, warmup):
    """Quality report of every decode matrix (w4a16_quant_error: its two
    kernels timed with HIP events, fp32 weights + packed bytes read), and the
    decode step through w4a16_linear_awq with 1 % of the input channels scaled
    by 8 (the decode kernel folds the activation scaling into its loads)."""
    import numpy as np
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl
    cfg = wl.WORKLOADS[HEADLINE]
    report = {}
    for j, mat in enumerate(cfg.matrices):
        w = torch.from_numpy(host_weights(HEADLINE, j)).to(dev)
        pw = w4.pack(w, cfg.group)
        r = w4.quant_error(w, pw)
        ws = w4.Workspace(dev)
        out = torch.empty(8, dtype=torch.float64, device=dev)
        for _ in range(20):
            w4.quant_error(w, pw, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record()
        for _ in range(reps):
            w4.quant_error(w, pw, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        assert out.cpu().tolist() == [r[f] for f in w4.QUALITY_FIELDS]   # deterministic
        nbytes = mat.N * mat.K * 4 + pw.nbytes()
        report[mat.name] = {"mse": r["mse"], "snr_db": round(r["snr_db"], 3), "cos": r["cos"],
                            "max_err": r["max_err"], "us": round(us, 1), "GBs": round(nbytes / us / 1e3, 1)}
        del w, pw
    torch.cuda.empty_cache()
    wk = Workload(HEADLINE, 1, dev)
    rng = np.random.default_rng(5)
    muls = []
    for m in wk.mats:
        a = np.ones(m.K, dtype=np.float32)
        a[rng.choice(m.K, m.K // 100, replace=False)] = 8.0
        muls.append(torch.from_numpy((1.0 / a).astype(np.float32)).to(dev))
    plain_ms = wk.time_fn(wk.step, steps, warmup)
    awq_ms = wk.time_fn(lambda c: wk.step_awq(c, muls), steps, warmup)
    awq = {"ms_per_step": round(awq_ms, 5), "plain_ms_per_step": round(plain_ms, 5),
           "value": round(sum(wk.bytes) / (awq_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
           "note": "decode step through w4a16_linear_awq (activation scaling folded into the decode kernel)"}
    del wk
    torch.cuda.empty_cache()
    return report, awq


def format_legs(dev, steps, warmup, launches):
    """The decode step and the prefill GEMM in each weight-format variant: step
    GB/s over its own algorithmic bytes, per-kernel rates against the peaks."""
    import torch

    import workloads as wl
    legs = []
    for fmt, group in FORMAT_LEGS:
        wk = Workload(HEADLINE, 1, dev, fmt, group)
        ms = wk.time_fn(wk.step, steps, warmup)
        per = [wk.kernel_us(j, launches) for j in range(len(wk.mats))]
        kernel_gbs = sum(wk.bytes) / (sum(per) * 1e-6) / 1e9
        weights = sum(m.N * m.K for m in wk.mats)
        leg = {"format": fmt, "group": group,
               "bits_per_weight": round(8 * (sum(wk.bytes) - sum(2 * (m.N + m.K) for m in wk.mats)) / weights, 4),
               "ms_per_step": round(ms, 5), "value": round(sum(wk.bytes) / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
               "decode_kernels": {"achieved": round(kernel_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                                  "us": {m.name: round(per[j], 2) for j, m in enumerate(wk.mats)}}}
        del wk
        torch.cuda.empty_cache()
        pcfg = WORKLOAD_IDS["prefill"]
        pk = Workload(pcfg, wl.WORKLOADS[pcfg].ms[0], dev, fmt, group)
        us = pk.kernel_us(0, launches)
        tf = pk.flops[0] / (us * 1e-6) / 1e12
        leg["prefill"] = {"M": pk.M, "kernel_us": round(us, 2), "achieved": round(tf, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        del pk
        torch.cuda.empty_cache()
        legs.append(leg)
    return legs


CROSSOVER_MS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 1024, 2048)
CROSSOVER_SHAPES = ((15360, 5120), (13824, 5120))   # fused QKV and FFN up of the 13B shapes, group 128


def time_launches(fn, copies, n):
    """Microseconds per launch of fn(copy, stream): one graph of n launches
    rotating over the weight copies, replayed after a 50 ms warm-up, HIP
    events around the timed replay."""
    import torch
    fn(0, None)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(n):
                fn(i % copies, cap)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def crossover(dev):
    """The batch-size crossover between the decode kernel (M <= 8), the
    small-batch matrix-core kernel and the tiled GEMM: each kernel that takes
    the shape, timed per launch (cold weights: copies past the MALL) at every
    M of CROSSOVER_MS on the fused-QKV (15360 x 5120) and FFN-up (13824 x 5120)
    shapes, fp16 and bf16, and whether w4a16_linear's choice is the fastest
    (within 3 %)."""
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl
    rows = []
    for (N, K) in CROSSOVER_SHAPES:
        w = torch.from_numpy(wl.random_weights(N + K, N, K)).to(dev)
        pw = w4.pack(w, 128)
        del w
        copies = max(1, -(-3 * MALL_BYTES // pw.nbytes()))
        sets = [pw] + [w4.PackedWeight(pw.qweight.clone(), pw.scales.clone(), pw.zeros.clone(), N, K, 128)
                       for _ in range(copies - 1)]
        for dtype in ("f16", "bf16"):
            tdt = torch.float16 if dtype == "f16" else torch.bfloat16
            for M in CROSSOVER_MS:
                x = torch.randn(M, K, device=dev).to(tdt)
                y = torch.empty(M, N, device=dev, dtype=tdt)
                kernels = (["gemv"] if M <= 8 else []) + (["small_batch"] if M <= 512 else []) + ["tiled"]
                times = {}
                for kname in kernels:
                    ws = w4.Workspace(dev)
                    n = 240 if M <= 64 else (120 if M <= 512 else 60)
                    times[kname] = round(time_launches(
                        lambda c, st: w4.linear_run(kname, x, sets[c], out=y, workspace=ws, stream=st), copies, n), 2)
                chosen = w4.linear_kernel(M, N, K, 128, tdt)
                best = min(times, key=times.get)
                rows.append({"N": N, "K": K, "dtype": dtype, "M": M, "us": times, "linear_chooses": chosen,
                             "fastest": best, "chosen_within_3pct": times[chosen] <= 1.03 * times[best]})
                print(f"N={N} K={K} {dtype} M={M}: " + " ".join(f"{k} {v:.2f}" for k, v in times.items()) +
                      f" | linear: {chosen}" + ("" if rows[-1]["chosen_within_3pct"] else "  (NOT the fastest)"),
                      file=sys.stderr, flush=True)
        del sets, pw
        torch.cuda.empty_cache()
    return rows


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_baseline(stash):
    """The oracle as it stands, timed on the host on sampled rows of every
    workload: quantise + pack (device layout) of those rows, then dequantise +
    fp64 product (and |x||w| product) for every batch size, timed separately;
    plus a one-thread pass of c1. The same results check the GPU: codes,
    scales and zero-points of the sampled rows bit for bit, outputs on them
    against the bar (bare, and with bf16's output rounding)."""
    import numpy as np

    import workloads as wl
    from oracle import w4a16_ref as ref
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
    except Exception:   # threadpoolctl missing: report the affinity count
        threadpool_limits = None
        blas_threads = len(os.sched_getaffinity(0))
    per_config = {}
    tot_bytes, tot_s = 0, 0.0
    for cfg_id in sorted({k[0] for k in stash}):
        cfg = wl.WORKLOADS[cfg_id]
        Ms = sorted(M for (c, M) in stash if c == cfg_id)
        t_quant = t_mm = 0.0
        work_bytes = work_flops = 0
        bitexact, worst_bare, worst_bar, rows_checked = True, 0.0, 0.0, 0
        for j, mat in enumerate(cfg.matrices):
            rows = stash[(cfg_id, Ms[0])]["results"][j]["rows"]
            w = host_weights(cfg_id, j)[rows]
            t1 = time.perf_counter()
            codes, s_bits, zeros = ref.quantize_groupwise(w, cfg.group)
            ref.pack_device(codes)
            ref.pack_scales_device(s_bits, cfg.group)
            ref.pack_zeros_device(zeros, cfg.group)
            t_quant += time.perf_counter() - t1
            for M in Ms:
                res = stash[(cfg_id, M)]["results"][j]
                exact = bool(np.array_equal(res["codes"], codes) and np.array_equal(res["s_bits"], s_bits)
                             and np.array_equal(res["zeros"], zeros))
                bitexact &= exact
                xb = stash[(cfg_id, M)]["x_bits"][j]
                t1 = time.perf_counter()
                w_hat = ref.dequantize(codes, s_bits, zeros, cfg.group)
                y_ref, a = ref.linear_ref(xb, cfg.dtype, w_hat)
                t_mm += time.perf_counter() - t1
                bare = float(ref.error_ratio(res["y"], y_ref, a).max())
                bar = float(ref.error_ratio(res["y"], y_ref, a, cfg.dtype).max())
                worst_bare, worst_bar = max(worst_bare, bare), max(worst_bar, bar)
                entry = stash[(cfg_id, M)]["entries"][mat.name]
                entry["max_err_ratio"] = round(bare, 4)
                entry["max_err_ratio_with_output_rounding"] = round(bar, 4)
                entry["codes_bitexact"] = exact
                entry["oracle_rows_checked"] = int(len(rows))
                work_bytes += algorithmic_bytes(M, len(rows), mat.K, cfg.group)
                work_flops += 2 * M * len(rows) * mat.K
            rows_checked += len(rows)
        per_config[f"c{cfg_id}"] = {
            "workload": cfg.name, "rows_per_matrix": int(len(rows)), "matrices": len(cfg.matrices), "Ms": Ms,
            "oracle_quant_s": round(t_quant, 3), "oracle_matmul_s": round(t_mm, 3),
            "quant_weights_per_s": round(rows_checked * cfg.matrices[0].K / max(t_quant, 1e-9)),
            "matmul_GBps": round(work_bytes / max(t_mm, 1e-9) / 1e9, 3),
            "matmul_GFLOPs": round(work_flops / max(t_mm, 1e-9) / 1e9, 3),
            "codes_scales_zeros_bitexact": bitexact, "max_err_ratio": round(worst_bare, 4),
            "max_err_ratio_with_output_rounding": round(worst_bar, 4)}
        tot_bytes += work_bytes
        tot_s += t_mm
    one = None
    if (1, 1) in stash and threadpool_limits is not None:
        res = stash[(1, 1)]["results"][0]
        cfg = wl.WORKLOADS[1]
        w = host_weights(1, 0)[res["rows"]]
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            codes, s_bits, zeros = ref.quantize_groupwise(w, cfg.group)
            ref.pack_device(codes)
            tq = time.perf_counter() - t1
            t1 = time.perf_counter()
            ref.linear_ref(stash[(1, 1)]["x_bits"][0], cfg.dtype, ref.dequantize(codes, s_bits, zeros, cfg.group))
            tm = time.perf_counter() - t1
        nb = algorithmic_bytes(1, len(res["rows"]), cfg.matrices[0].K, cfg.group)
        one = {"threads": 1, "oracle_quant_s": round(tq, 3), "oracle_matmul_s": round(tm, 3),
               "matmul_GBps": round(nb / tm / 1e9, 3)}
    return {"value": round(tot_bytes / max(tot_s, 1e-9) / 1e9, 3), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle", "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "threads": {"quantise_pack": 1, "dequantise": 1, "fp64_product": blas_threads},
            "sample": "sampled rows (output columns) of every matrix of every workload: quantise + pack in numpy "
                      "(one thread), dequantise (numpy, one thread) + fp64 products x.w_hat^T and |x|.|w_hat|^T "
                      f"(BLAS, {blas_threads} threads) at every batch size; value = algorithmic bytes of those rows "
                      "over the dequantise + product time",
            "per_config": per_config, "one_thread_c1": one}


def device_info(dev):
    import torch
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__}


# ---------------------------------------------------------------------------
# profiling support: the counter pass and the summaries of rocprofv3 output
# ---------------------------------------------------------------------------

def counter_pass(out_dir, reps, legs):
    """Each matrix of each leg launched `reps` times eagerly (copies rotated),
    in an order written to out_dir/counter_pass.json, after one 256 MiB copy
    (w4a16_measure_copy: 256 MiB read, 256 MiB written) that scales the
    counters."""
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl
    dev = torch.device("cuda:0")
    os.makedirs(out_dir, exist_ok=True)
    seq = []
    src = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    assert w4.raw().w4a16_measure_copy(src.data_ptr(), dst.data_ptr(), CALIBRATION_BYTES, None) == 0
    torch.cuda.synchronize()
    seq.append({"kernel": "copy_kernel", "bytes_read": CALIBRATION_BYTES, "bytes_written": CALIBRATION_BYTES,
                "launches": 1})
    del src, dst
    for cfg_id in legs:
        for M in wl.WORKLOADS[cfg_id].ms:
            wk = Workload(cfg_id, M, dev)
            for j, m in enumerate(wk.mats):
                for i in range(reps):
                    wk.launch(i % wk.copies, j)
                torch.cuda.synchronize()
                seq.append({"workload": wk.cfg.name, "M": M, "matrix": m.name, "N": m.N, "K": m.K,
                            "bytes_algorithmic": wk.bytes[j], "flops": wk.flops[j], "launches": reps,
                            "kernel_source_sha": kernel_source_hash(wk.launch_keys[j]["kind"]),
                            **wk.launch_keys[j]})
            del wk
            torch.cuda.empty_cache()
            print(f"counter pass: {wl.WORKLOADS[cfg_id].name} M={M} done", flush=True)
    json.dump(seq, open(os.path.join(out_dir, "counter_pass.json"), "w"), indent=1)


def _csv_rows(directory, suffix):
    """Rows of every rocprofv3 CSV file (plain or gzipped) named *suffix under directory."""
    import gzip
    rows = []
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    files += glob.glob(os.path.join(directory, "**", f"*{suffix}.gz"), recursive=True)
    for f in sorted(files):
        with (gzip.open(f, "rt") if f.endswith(".gz") else open(f)) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    """Kernel name without return type, namespaces and parameter list."""
    name = name.replace("w4a16::", "").replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*$", "", name)[:70]


LIBRARY_KERNELS = ("decode_kernel", "decode_bcast_kernel", "decode_group_kernel", "skinny_kernel",
                   "skinny_group_kernel", "prefill_kernel", "copy_kernel", "stream_read_kernel")


def _int(r, *keys):
    for k in keys:
        if r.get(k) not in (None, ""):
            return int(float(r[k]))
    return 0


def _template_args(name):
    m = re.search(r"<(.*)>", name)
    return [a.strip() for a in m.group(1).split(",")] if m else []


def _matches_leg(name, e, group, dtype):
    """Whether a trace row's kernel is the instantiation a bench entry ran:
    the 4-bit zero-point format (0) in the leg's group and activation type."""
    base, args = name.split("<")[0], _template_args(name)
    bf = "true" if dtype == "bf16" else "false"
    if base != e["kernel"] or not args:
        return False
    if base == "decode_kernel":       # <GROUP, MT, BF, FMT, NCOL, AWQ>
        return args[0] == str(group) and args[2] == bf and args[3] == "0" and args[5] == "false"
    if base == "decode_bcast_kernel":  # <GROUP, BF, FMT, NCOL, D>
        return args[0] == str(group) and args[1] == bf and args[2] == "0"
    if base == "skinny_kernel":       # <GROUP, R, BF, FMT>
        return args[0] == str(group) and args[2] == bf and args[3] == "0"
    if base == "prefill_kernel":      # <BM, BN, WM, WN, GROUP, BF, FMT, SK>
        return args[4] == str(min(group, 128)) and args[5] == bf and args[6] == "0"
    return False


def summarize_trace(directory, bench_json):
    """Kernel trace (rocprofv3 --kernel-trace --output-format csv): launches per
    (kernel instantiation, workgroups, threads) with median / p10 / p90 / mean
    duration; with a bench.py output line, the legs' matrices whose launch
    (kernel, format, group, type and geometry) a row matches are listed under
    it with the bench's per-launch time."""
    groups = {}
    for r in _csv_rows(directory, "kernel_trace.csv"):
        name = _short(r["Kernel_Name"])
        if name.split("<")[0] not in LIBRARY_KERNELS:
            continue
        wg_size = _int(r, "Workgroup_Size_X", "Workgroup_Size")
        grid = _int(r, "Grid_Size_X", "Grid_Size")
        key = (name, grid // max(wg_size, 1), wg_size)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    entries = []
    if bench_json:
        b = json.loads(open(bench_json).read().strip().splitlines()[-1])
        for leg in b.get("legs", {}).values():
            for M, ents in leg["by_M"].items():
                for mname, e in ents.items():
                    entries.append((f"{leg['workload']} M={M} {mname}", e, leg["group"], leg["dtype"]))
    lines = [f"{'kernel':<62} {'wgs':>6} {'thr':>4} {'n':>6} {'median_us':>10} {'p10':>8} {'p90':>8} {'mean':>8}"]
    for (name, wgs, thr), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d.sort()
        q = lambda f: d[min(len(d) - 1, int(f * len(d)))]  # noqa: E731
        med = statistics.median(d)
        lines.append(f"{name:<62} {wgs:>6} {thr:>4} {len(d):>6} {med:>10.2f} {q(0.1):>8.2f} "
                     f"{q(0.9):>8.2f} {statistics.fmean(d):>8.2f}")
        for label, e, group, dtype in entries:
            if e["workgroups"] == wgs and e["threads"] == thr and _matches_leg(name, e, group, dtype):
                lines.append(f"    {label}: bench {e['us']:.2f} us per launch (events, dispatch gap included), "
                             f"{e['us'] / med:.3f} x the trace median")
    return "\n".join(lines)


def summarize_counters(directories):
    """Counter runs (rocprofv3 --pmc ... --output-format csv) of `bench.py
    --counter-pass`: the library's dispatches in order, matched to the pass's
    sequence; per matrix the median counter value per dispatch. FETCH_SIZE and
    WRITE_SIZE are scaled by the copy kernel's (256 MiB each way) and reported
    as bytes beside the algorithmic bytes."""
    seq = None
    per = {}
    for d in directories:
        sfile = glob.glob(os.path.join(d, "**", "counter_pass.json"), recursive=True)
        if sfile and seq is None:
            seq = json.load(open(sfile[0]))
        disp = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            name = _short(r["Kernel_Name"])
            if name.split("<")[0] not in LIBRARY_KERNELS:
                continue
            did = _int(r, "Dispatch_Id", "Correlation_Id")
            disp.setdefault(did, {"name": name, "c": {}})
            cn = r["Counter_Name"]
            disp[did]["c"][cn] = disp[did]["c"].get(cn, 0.0) + float(r["Counter_Value"])
        per[d] = [disp[k] for k in sorted(disp)]
    assert seq is not None, "no counter_pass.json found"
    table = []
    for d, dispatches in per.items():
        i = 0
        for s in seq:
            chunk = dispatches[i:i + s["launches"]]
            i += s["launches"]
            assert all(c["name"].split("<")[0] == s["kernel"] for c in chunk), (s, [c["name"] for c in chunk])
            label = "calibration copy" if s["kernel"] == "copy_kernel" else f"{s['workload']} M={s['M']} {s['matrix']}"
            ent = next((t for t in table if t["label"] == label), None)
            if ent is None:
                ent = {"label": label, "seq": s, "kernel": chunk[0]["name"], "counters": {}}
                table.append(ent)
            for c in chunk[0]["c"]:
                ent["counters"][c] = statistics.median(x["c"][c] for x in chunk)
        assert i == len(dispatches), f"{d}: {len(dispatches)} dispatches, the sequence has {i}"
    cal = next(t for t in table if t["label"] == "calibration copy")["counters"]
    scale = {}
    if "FETCH_SIZE" in cal:
        scale["FETCH_SIZE"] = CALIBRATION_BYTES / 1024 / cal["FETCH_SIZE"]
    if "WRITE_SIZE" in cal:
        scale["WRITE_SIZE"] = CALIBRATION_BYTES / 1024 / cal["WRITE_SIZE"]
    for t in table:
        c = t["counters"]
        if "FETCH_SIZE" in c:
            t["fetch_bytes"] = c["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        if "WRITE_SIZE" in c:
            t["write_bytes"] = c["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
    return table, scale


def write_traffic_json(table, scale, command):
    """profiles/traffic_<workload>_m<M>.json for every leg: HBM bytes of one
    launch of each matrix and of the whole set, read by the bench's `traffic`."""
    by_leg = {}
    for t in table:
        s = t["seq"]
        if s["kernel"] == "copy_kernel" or "fetch_bytes" not in t or "write_bytes" not in t:
            continue
        by_leg.setdefault((s["workload"], s["M"]), []).append(t)
    for (wname, M), ents in by_leg.items():
        kinds = sorted({e["seq"]["kind"] for e in ents})
        total = sum(e["fetch_bytes"] + e["write_bytes"] for e in ents)
        alg = sum(e["seq"]["bytes_algorithmic"] for e in ents)
        doc = {"command": command, "counter_scale": {k: round(v, 4) for k, v in scale.items()},
               "scale_from": "w4a16_measure_copy of 256 MiB (256 MiB read, 256 MiB written) in the same run",
               "workload": wname, "M": M, "kernel_kinds": kinds,
               "kernel_source_sha": ents[0]["seq"]["kernel_source_sha"] if len(kinds) == 1 else None,
               "traffic_bytes_per_launch_set": round(total),
               "algorithmic_bytes_per_launch_set": alg, "ratio_to_algorithmic": round(total / alg, 4),
               "per_matrix": {e["seq"]["matrix"]: {"kernel": e["kernel"], "fetch_bytes": round(e["fetch_bytes"]),
                                                   "write_bytes": round(e["write_bytes"]),
                                                   "algorithmic_bytes": e["seq"]["bytes_algorithmic"]}
                              for e in ents}}
        with open(os.path.join(ROOT, "profiles", f"traffic_{wname}_m{M}.json"), "w") as fh:
            json.dump(doc, fh, indent=1)


def print_counter_summary(table, scale, simds=1024, xcds=8):
    counters = sorted({c for t in table for c in t["counters"]})
    for t in table:
        c = t["counters"]
        # derived: share of the kernel's cycles the matrix cores were busy,
        # SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) / (busy cycles of one XCD x SIMDs);
        # rocprofv3 reports GRBM_GUI_ACTIVE summed over the XCDs
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            c["mfma_busy_pct"] = 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / xcds * simds)
        if "SQ_WAIT_ANY" in c and c.get("SQ_BUSY_CYCLES"):
            c["wait_any_per_busy"] = c["SQ_WAIT_ANY"] / c["SQ_BUSY_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_INSTS_LDS"):
            c["lds_conflict_per_inst"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"]
    counters = sorted({c for t in table for c in t["counters"]})
    if scale:
        print("counter scale (copy kernel): " + ", ".join(f"{k} x{v:.4f}" for k, v in scale.items()))
    print(f"{'launch':<34} {'kernel':<44} " + " ".join(f"{c:>24}" for c in counters) +
          ("  fetch_MB write_MB alg_MB ratio" if scale else ""))
    for t in table:
        s = t["seq"]
        alg = s.get("bytes_algorithmic", s.get("bytes_read", 0) + s.get("bytes_written", 0))
        tot = t.get("fetch_bytes", 0) + t.get("write_bytes", 0)
        extra = ""
        if "fetch_bytes" in t or "write_bytes" in t:
            extra = (f"  {t.get('fetch_bytes', 0) / 1e6:8.2f} {t.get('write_bytes', 0) / 1e6:8.2f} {alg / 1e6:6.2f} "
                     f"{tot / alg:5.3f}")
        print(f"{t['label']:<34} {t['kernel'][:44]:<44} " +
              " ".join(f"{t['counters'].get(c, float('nan')):>24.2f}" for c in counters) + extra)


def main():
    args = parse()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.bench_json))
        return
    if args.summarize_counters:
        table, scale = summarize_counters(args.summarize_counters)
        print_counter_summary(table, scale)
        if "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
            write_traffic_json(table, scale, "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE, separate runs) "
                                             "--output-format csv -- python3 bench.py --counter-pass DIR")
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding of the layer is described, not built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    assert w4.device_supported(0), "cuda:0 is not a gfx950"
    w4.init(0)
    launches = max(200, args.launches)
    legs_ids = [int(v) for v in args.legs.split(",") if v]

    if args.counter_pass:
        counter_pass(args.counter_pass, args.reps, legs_ids)
        return

    if args.stream_grid:
        print(json.dumps({"stream_grid": stream_grid(dev), "device": device_info(dev)}))
        return

    if args.crossover:
        rows = crossover(dev)
        print(json.dumps({"crossover": rows, "all_chosen_within_3pct": all(r["chosen_within_3pct"] for r in rows),
                          "device": device_info(dev)}))
        return

    if args.workload:   # one workload's leg only (batch sweeps): no headline, no oracle
        cfg_id = WORKLOAD_IDS[args.workload]
        Ms = [args.m] if args.m else list(wl.WORKLOADS[cfg_id].ms)
        leg = run_leg(cfg_id, Ms, dev, launches, None)
        print(json.dumps({"workload": args.workload, "leg": leg, "device": device_info(dev)}))
        return

    stash = {}
    step, c2_entries, grouped = headline(dev, args.steps, args.warmup, launches, stash)
    print(f"headline step {step['ms_per_step'] * 1e3:.2f} us", file=sys.stderr, flush=True)
    legs = {"c2": {"workload": wl.WORKLOADS[HEADLINE].name, "group": wl.WORKLOADS[HEADLINE].group, "dtype": "f16",
                   "seeds": "numpy default_rng([2, matrix, 0]) weights, ([2, matrix, 1, M]) activations",
                   "by_M": {"1": c2_entries}}}
    for cfg_id in legs_ids:
        if cfg_id == HEADLINE:
            continue
        legs[f"c{cfg_id}"] = run_leg(cfg_id, list(wl.WORKLOADS[cfg_id].ms), dev, launches, stash)
        print(f"leg c{cfg_id} done", file=sys.stderr, flush=True)
    # the streaming read beside every M = 1 decode launch: the headline set, c1 and c5
    ceiling_entries = dict(c2_entries)
    for cid, mat in (("c1", "w"), ("c5", "down")):
        e = legs.get(cid, {}).get("by_M", {}).get("1", {}).get(mat)
        if e is not None and e.get("kind") == "gemv":
            ceiling_entries[f"{cid}_{mat}"] = e
    ceiling = stream_ceiling(dev, ceiling_entries)

    # ---- the dominant kernel of the headline step
    by_kind = {}
    for e in c2_entries.values():
        k = by_kind.setdefault(e["kernel"], {"us": 0.0, "bytes": 0, "launches": 0, "kind": e["kind"]})
        k["us"] += e["us"]
        k["bytes"] += e["bytes_algorithmic"]
        k["launches"] += 1
    dom = max(by_kind, key=lambda k: by_kind[k]["us"])
    d = by_kind[dom]
    gbs = d["bytes"] / (d["us"] * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(wl.WORKLOADS[HEADLINE].name, 1, d["kind"]),
            "kernel": dom, "launches_per_step": d["launches"], "kernel_source_sha": kernel_source_hash(d["kind"]),
            "timing": f"HIP events on the replay stream around {launches} back-to-back launches per matrix "
                      "(dispatch gap included)",
            "units_per_launch": {n: {"weights": e["N"] * e["K"], "bytes": e["bytes_algorithmic"], "us": e["us"]}
                                 for n, e in c2_entries.items()}}

    prefill = None
    if "c4" in legs:
        e = legs["c4"]["by_M"]["2048"]["up"]
        prefill = {"workload": "prefill", "M": 2048, "N": e["N"], "K": e["K"], "kernel": e["kernel"],
                   "kernel_us": e["us"], "tflops": e["TFLOPs"], "tokens_per_s": e["tokens_per_s"],
                   "roofline": {"bound": "mfma", "achieved": e["TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(e["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                                "traffic": stored_traffic("prefill", 2048, e["kind"]),
                                "kernel_source_sha": kernel_source_hash(e["kind"])}}

    quality = awq = formats = None
    if not args.no_formats:
        quality, awq = quality_and_awq(dev, max(200, args.steps // 2), args.warmup)
        formats = format_legs(dev, max(200, args.steps // 2), args.warmup, launches)

    cpu = None if args.no_cpu_baseline else cpu_oracle_baseline(stash)

    value = step["bytes"] / (step["ms_per_step"] * 1e-3) / 1e9
    out = {
        "metric": "W4A16 GEMV achieved HBM GB/s (% peak) at M=1; GEMM TFLOP/s (% MFMA) at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step["ms_per_step"], 5),
        "gpu_ms_per_step": round(step["gpu_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.WORKLOADS[HEADLINE].name, "M": 1, "group": wl.WORKLOADS[HEADLINE].group,
                   "matrices": [[m.name, m.N, m.K] for m in wl.WORKLOADS[HEADLINE].matrices],
                   "bytes_per_step": step["bytes"], "flops_per_step": step["flops"]},
        "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "tokens_per_s": round(1 / (step["ms_per_step"] * 1e-3), 1),
        "roofline": roof,
        "legs": legs,
        "stream_ceiling": ceiling,
        "grouped_step": grouped,
        "prefill": prefill,
        "formats": formats,
        "quality": quality,
        "awq_step": awq,
        "cpu_baseline": cpu,
        "device": device_info(dev),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
