#!/usr/bin/env python3
"""Benchmark of the gfx950 W4A16 linear layer.

Headline workload (default): the decode layer set of a 13B-class model at
M = 1 -- q, k, v, o (K = N = 5120), up and gate (K = 5120, N = 13824), down
(K = 13824, N = 5120), group 128, fp16 activations. One step = one token
through all seven layers (seven w4a16_linear calls, dispatched to the decode
GEMV at M = 1). Second leg: the prefill GEMM, M = 2048, K = 5120, N = 13824,
group 128, bf16 activations (w4a16_linear dispatches to the tiled MFMA kernel).

Inputs are synthetic and seeded; packed weights are rotated over enough copies
to exceed the 256 MB last-level cache, so every launch streams its weights
from HBM. Launches are replayed from HIP graphs.

Prints one JSON line. `value` is achieved HBM GB/s of the headline step
(algorithmic bytes -- packed weights + scales + zeros + activations read +
outputs written -- over wall time per step). `roofline` is the decode GEMV
kernel's own rate: algorithmic bytes of its launches over their average
duration from HIP events on the launch stream. `prefill` carries the M = 2048
GEMM's TFLOP/s against the dense bf16 MFMA peak. `grouped_step` times the same
seven layers with q/k/v and gate/up each in one launch (w4a16_linear_group);
`value` stays the seven-launch step. `formats` repeats the decode step and
the prefill GEMM with the weights in the other formats (symmetric 4-bit,
symmetric 8-bit = W8A16, group 256, K-quant-style super-blocks), each against
its own bytes and flops.
`quality` is the quantisation quality report of each matrix (w4a16_quant_error)
and `awq_step` the decode step through the AWQ run-time path.
`cpu_baseline` times the CPU
oracle (dequantise + fp64 product) on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA
MALL_BYTES = 256 << 20
WORKLOAD_IDS = {"gemv_4096": 1, "decode_13b_layer": 2, "fused_qkv": 3, "prefill": 4, "ffn_down_70b": 5}

# sources each kernel is built from (for matching stored counter results)
KERNEL_SOURCES = {
    "gemv": ["decode.hip", "decode_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
    "skinny": ["gemm.hip", "gemm_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
    "prefill": ["prefill.hip", "prefill_kernel.hpp", "decode_common.hpp", "w4a16_internal.hpp"],
}
# weight-format variants measured beside the headline (format, group)
FORMAT_LEGS = [("sym4", 128), ("sym8", 128), ("asym4", 256), ("kq4", 256)]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--workload", default="decode_13b_layer", choices=list(WORKLOAD_IDS))
    p.add_argument("--m", type=int, default=0, help="batch rows (default: the workload's first M)")
    p.add_argument("--no-prefill", action="store_true", help="skip the M=2048 prefill leg")
    p.add_argument("--prefill-reps", type=int, default=600,
                   help="prefill launches timed (about 170 ms at M=2048), after a quarter as many untimed")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-formats", action="store_true", help="skip the weight-format legs")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run an elementwise kernel that reads and writes 256 MiB (counter scaling)")
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


def algorithmic_bytes(M, N, K, group, fmt="asym4"):
    """Codes (4 or 8 bits per weight), fp16 scales, 4-bit zero-points (asym4
    only), activations read and outputs written."""
    G = K // group
    codes = N * K if fmt == "sym8" else N * K // 2
    zeros = G * N // 2 if fmt == "asym4" else 0
    meta = 16 * (K // 256) * N if fmt == "kq4" else 2 * G * N    # kq4: 16-byte super-block records
    return codes + meta + zeros + 2 * M * K + 2 * M * N


def kernel_kind(w4, M, N, K, group, dtype):
    """Kernel w4a16_linear uses for this shape (as the library reports it)."""
    import torch
    k = w4.linear_kernel(M, N, K, group, torch.bfloat16 if dtype == "bf16" else torch.float16)
    return {"gemv": "gemv", "small_batch": "skinny", "tiled": "prefill"}[k]


def stored_traffic(workload, M, kind):
    """HBM bytes per step from committed counter runs, if taken on these sources."""
    tfile = os.path.join(ROOT, "profiles", f"traffic_{workload}_m{M}.json")
    if not os.path.exists(tfile):
        return None
    t = json.load(open(tfile))
    if t.get("kernel_source_sha") != kernel_source_hash(kind):
        return None
    return t.get("traffic_bytes_per_launch_set")


class Workload:
    """Packed weights, activations and outputs of one configuration, with
    enough rotated copies of the weights to defeat the 256 MB MALL."""

    def __init__(self, cfg_id, M, dev, fmt="asym4", group=None):
        import numpy as np
        import torch

        import w4a16_weight_only_dequant_amd as w4
        import workloads as wl
        self.w4, self.torch = w4, torch
        self.cfg = wl.WORKLOADS[cfg_id]
        self.M, self.group, self.dtype = M, group or self.cfg.group, self.cfg.dtype
        self.fmt = fmt
        tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        self.mats = list(self.cfg.matrices)
        packed, self.xs, self.ys = [], [], []
        for mi, mat in enumerate(self.mats):
            w = torch.from_numpy(wl.weights(cfg_id, mi)).to(dev)
            packed.append(w4.pack(w, self.group, fmt))
            del w
            xb = wl.activations(cfg_id, mi, M)
            self.xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(tdt))
            self.ys.append(torch.empty((M, mat.N), dtype=tdt, device=dev))
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

    def time_grouped(self, dev, groups, steps, warmup):
        """Wall time per step of the grouped step (one HIP graph per weight copy)."""
        return self.time_fn(dev, lambda c: self.step_grouped(c, groups), steps, warmup)

    def step_awq(self, c, act_mul):
        """One step through w4a16_linear_awq (activation multipliers per matrix)."""
        for j in range(len(self.mats)):
            self.w4.linear_awq(self.xs[j], act_mul[j], self.sets[c][j], out=self.ys[j], workspace=self.ws)

    def time_fn(self, dev, fn, steps, warmup):
        """Wall time per step of fn(copy) replayed from one HIP graph per weight copy."""
        torch = self.torch
        for c in range(min(2, self.copies)):
            fn(c)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream(device=dev)
        graphs = []
        with torch.cuda.stream(cap):
            for c in range(self.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    fn(c)
                graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % self.copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % self.copies].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def graphs(self, dev):
        """One graph per weight copy holding one step; one graph per matrix
        holding that matrix's launch on every copy (per-kernel timing)."""
        torch = self.torch
        for c in range(min(2, self.copies)):
            self.step(c)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream(device=dev)
        self.step_graphs, self.mat_graphs = [], []
        with torch.cuda.stream(cap):
            for c in range(self.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    self.step(c)
                self.step_graphs.append(g)
            for j in range(len(self.mats)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for c in range(self.copies):
                        self.launch(c, j)
                self.mat_graphs.append(g)
        torch.cuda.synchronize()

    def per_kernel_ms(self, reps):
        """Average duration of one launch per matrix: HIP events on the
        replay stream around back-to-back launches (the gap between two
        dependent launches is included), after a quarter as many untimed
        replays: the device's clocks take milliseconds to rise under a new
        load (M = 2048 prefill: 318 us per launch over the first 7 ms, 280 us
        sustained)."""
        torch = self.torch
        out = []
        for j in range(len(self.mats)):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            for _ in range(max(1, reps // 4)):
                self.mat_graphs[j].replay()
            a0.record()
            for _ in range(reps):
                self.mat_graphs[j].replay()
            a1.record()
            torch.cuda.synchronize()
            out.append(a0.elapsed_time(a1) / (reps * self.copies))
        return out


def cpu_oracle_baseline(cfg_id, M, seconds):
    """The oracle as it stands, timed on the host: dequantise + fp64 product,
    matrix by matrix, until about `seconds` of CPU work is done."""
    import workloads as wl
    from oracle import w4a16_ref as ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
    except Exception:   # threadpoolctl missing: report the affinity count
        blas_threads = len(os.sched_getaffinity(0))
    cfg = wl.WORKLOADS[cfg_id]
    mats = list(cfg.matrices)
    done_bytes, t_cpu, names, mi = 0, 0.0, [], 0
    prepared = {}
    while t_cpu < seconds and mi < 40 * len(mats):
        j = mi % len(mats)
        if j not in prepared:   # offline quantisation, untimed, once per matrix
            prepared[j] = (ref.quantize_groupwise(wl.weights(cfg_id, j), cfg.group), wl.activations(cfg_id, j, M))
        (codes, s_bits, zeros), xb = prepared[j]
        t1 = time.perf_counter()
        w_hat = ref.dequantize(codes, s_bits, zeros, cfg.group)
        ref.linear_ref(xb, cfg.dtype, w_hat)
        t_cpu += time.perf_counter() - t1
        done_bytes += algorithmic_bytes(M, mats[j].N, mats[j].K, cfg.group)
        names.append(mats[j].name)
        mi += 1
        del w_hat
    return {"value": round(done_bytes / t_cpu / 1e9, 3), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": f"dequantise (numpy, one thread) + fp64 product and |x||w| product (BLAS, "
                      f"{blas_threads} threads) of {len(names)} matrix launches of the workload "
                      f"({','.join(names[:len(mats)])}, repeated) at M={M}: "
                      f"{done_bytes / 1e6:.0f} MB of its algorithmic bytes in {t_cpu:.1f} s"}


def time_steps(wk, steps, warmup):
    """Wall time per step of replaying the step graphs (weights rotated over copies)."""
    torch = wk.torch
    for i in range(warmup):
        wk.step_graphs[i % wk.copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        wk.step_graphs[i % wk.copies].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def quality_and_awq(dev, cfg_id, M, steps, warmup):
    """Quality report of every matrix of the workload (w4a16_quant_error: its
    two kernels timed with HIP events, fp32 weights + packed bytes read), and
    the decode step through w4a16_linear_awq with 1 % of the input channels
    scaled by 8 (the GEMV folds the activation scaling into its staging)."""
    import numpy as np
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl
    cfg = wl.WORKLOADS[cfg_id]
    report = {}
    for j, mat in enumerate(cfg.matrices):
        w = torch.from_numpy(wl.weights(cfg_id, j)).to(dev)
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
        us = e0.elapsed_time(e1) * 1e3 / reps   # the two kernels back to back, no host copy
        assert out.cpu().tolist() == [r[f] for f in w4.QUALITY_FIELDS]   # deterministic
        nbytes = mat.N * mat.K * 4 + pw.nbytes()
        report[mat.name] = {"mse": r["mse"], "snr_db": round(r["snr_db"], 3), "cos": r["cos"],
                            "max_err": r["max_err"], "us": round(us, 1), "GBs": round(nbytes / us / 1e3, 1)}
        del w, pw
    torch.cuda.empty_cache()
    wk = Workload(cfg_id, M, dev)
    rng = np.random.default_rng(5)
    muls = []
    for m in wk.mats:
        a = np.ones(m.K, dtype=np.float32)
        a[rng.choice(m.K, m.K // 100, replace=False)] = 8.0
        muls.append(torch.from_numpy((1.0 / a).astype(np.float32)).to(dev))
    plain_ms = wk.time_fn(dev, wk.step, steps, warmup)
    awq_ms = wk.time_fn(dev, lambda c: wk.step_awq(c, muls), steps, warmup)
    awq = {"ms_per_step": round(awq_ms, 5), "plain_ms_per_step": round(plain_ms, 5),
           "value": round(sum(wk.bytes) / (awq_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
           "note": "decode step through w4a16_linear_awq (activation scaling folded into the GEMV staging)"}
    del wk
    torch.cuda.empty_cache()
    return report, awq


def format_legs(dev, cfg_id, M, steps, warmup, prefill_reps):
    """The decode step and the prefill GEMM in each weight-format variant: step
    GB/s over its own algorithmic bytes, per-kernel rates against the peaks."""
    import workloads as wl
    torch = __import__("torch")
    legs = []
    for fmt, group in FORMAT_LEGS:
        wk = Workload(cfg_id, M, dev, fmt, group)
        wk.graphs(dev)
        ms = time_steps(wk, steps, warmup)
        per = wk.per_kernel_ms(max(1, steps // (wk.copies * 4)))
        kernel_gbs = sum(wk.bytes) / (sum(per) * 1e-3) / 1e9
        leg = {"format": fmt, "group": group, "bits_per_weight": round(8 * (sum(wk.bytes) - sum(
                   2 * M * (m.N + m.K) for m in wk.mats)) / sum(m.N * m.K for m in wk.mats), 4),
               "ms_per_step": round(ms, 5), "value": round(sum(wk.bytes) / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
               "decode_kernels": {"achieved": round(kernel_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                                  "us": {m.name: round(per[j] * 1e3, 2) for j, m in enumerate(wk.mats)}}}
        del wk
        torch.cuda.empty_cache()
        pcfg = WORKLOAD_IDS["prefill"]
        pk = Workload(pcfg, wl.WORKLOADS[pcfg].ms[0], dev, fmt, group)
        pk.graphs(dev)
        pms = pk.per_kernel_ms(max(1, prefill_reps // pk.copies))
        tf = pk.flops[0] / (pms[0] * 1e-3) / 1e12
        leg["prefill"] = {"M": pk.M, "kernel_us": round(pms[0] * 1e3, 2), "achieved": round(tf, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        del pk
        torch.cuda.empty_cache()
        legs.append(leg)
    return legs


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding of the layer is described, not built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import w4a16_weight_only_dequant_amd as w4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    assert w4.device_supported(0), "cuda:0 is not a gfx950"

    import workloads as wl
    cfg_id = WORKLOAD_IDS[args.workload]
    M = args.m or wl.WORKLOADS[cfg_id].ms[0]
    wk = Workload(cfg_id, M, dev)
    wk.graphs(dev)
    for i in range(args.warmup):
        wk.step_graphs[i % wk.copies].replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, bracketed by synchronisation ----
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        wk.step_graphs[i % wk.copies].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    step_bytes, step_flops = sum(wk.bytes), sum(wk.flops)

    # ---- the dominant kernel's own rate: the kernel with the most time in
    # the step, its algorithmic bytes (or flops) over its launches' durations
    per_ms = wk.per_kernel_ms(max(1, args.steps // (wk.copies * 4)))
    kinds = [kernel_kind(w4, M, m.N, m.K, wk.group, wk.dtype) for m in wk.mats]
    by_kind = {}
    for j, k in enumerate(kinds):
        e = by_kind.setdefault(k, {"ms": 0.0, "bytes": 0, "flops": 0, "launches": 0})
        e["ms"] += per_ms[j]
        e["bytes"] += wk.bytes[j]
        e["flops"] += wk.flops[j]
        e["launches"] += 1
    names = {"gemv": "gemv_kernel", "skinny": "skinny_kernel", "prefill": "prefill_kernel"}

    def roofline(kind, e):
        if kind == "prefill":
            tf = e["flops"] / (e["ms"] * 1e-3) / 1e12
            return {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        gbs = e["bytes"] / (e["ms"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}

    kind = max(by_kind, key=lambda k: by_kind[k]["ms"])
    roof = roofline(kind, by_kind[kind])
    roof["traffic"] = stored_traffic(args.workload, M, kind)
    roof["kernel"] = names[kind]
    roof["launches_per_step"] = by_kind[kind]["launches"]
    roof["kernel_source_sha"] = kernel_source_hash(kind)
    roof["timing"] = "HIP events on the replay stream around back-to-back launches of one matrix"
    roof["by_kernel"] = {names[k]: dict(roofline(k, e), launches=e["launches"], us=round(e["ms"] * 1e3, 2))
                         for k, e in by_kind.items()}
    roof["units_per_launch"] = {m.name: {"kernel": names[kinds[j]], "weights": m.N * m.K, "bytes": wk.bytes[j],
                                         "kernel_us": round(per_ms[j] * 1e3, 2)}
                                for j, m in enumerate(wk.mats)}
    # ---- the same step with the independent layers of one token grouped in
    # one launch each (w4a16_linear_group): q, k, v share their input in a
    # model, so do gate and up; o and down each follow a dependency
    grouped = None
    if args.workload == "decode_13b_layer":
        names_idx = {m.name: j for j, m in enumerate(wk.mats)}
        groups = [[names_idx[n] for n in g] for g in (("q", "k", "v"), ("o",), ("up", "gate"), ("down",))]
        g_ms = wk.time_grouped(dev, groups, args.steps, args.warmup)
        g_val = step_bytes / (g_ms * 1e-3) / 1e9
        grouped = {"ms_per_step": round(g_ms, 5), "value": round(g_val, 1), "unit": "GB/s",
                   "pct_hbm_peak": round(g_val / HBM_PEAK_GBS * 100, 2), "launches_per_step": len(groups),
                   "groups": [[wk.mats[j].name for j in g] for g in groups],
                   "tokens_per_s": round(M / (g_ms * 1e-3), 1)}
    del wk
    torch.cuda.empty_cache()

    # ---- prefill leg: M = 2048 GEMM (MFMA) ----
    prefill = None
    if not args.no_prefill and args.workload != "prefill":
        pk = Workload(WORKLOAD_IDS["prefill"], wl.WORKLOADS[WORKLOAD_IDS["prefill"]].ms[0], dev)
        pk.graphs(dev)
        pms = pk.per_kernel_ms(max(1, args.prefill_reps // pk.copies))
        pkind = kernel_kind(w4, pk.M, pk.mats[0].N, pk.mats[0].K, pk.group, pk.dtype)
        tf = pk.flops[0] / (pms[0] * 1e-3) / 1e12
        prefill = {"workload": "prefill", "M": pk.M, "N": pk.mats[0].N, "K": pk.mats[0].K, "group": pk.group,
                   "dtype": pk.dtype, "kernel": "prefill_kernel" if pkind == "prefill" else pkind,
                   "kernel_us": round(pms[0] * 1e3, 2), "tflops": round(tf, 1),
                   "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                "traffic": stored_traffic("prefill", pk.M, pkind),
                                "kernel_source_sha": kernel_source_hash(pkind)},
                   "tokens_per_s": round(pk.M / (pms[0] * 1e-3), 1)}
        del pk
        torch.cuda.empty_cache()

    quality, awq = None, None
    if not args.no_formats and args.workload == "decode_13b_layer":
        quality, awq = quality_and_awq(dev, cfg_id, M, max(20, args.steps // 2), args.warmup)

    formats = None
    if not args.no_formats:
        formats = format_legs(dev, cfg_id, M, max(20, args.steps // 2), args.warmup, args.prefill_reps // 2)

    if args.copy_calibration:
        # an elementwise kernel of known traffic (reads 256 MiB, writes 256 MiB):
        # counter bytes of this launch give the scale factor for the others
        a = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 2.0, out=b)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_baseline(cfg_id, M, args.cpu_seconds)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "W4A16 GEMV achieved HBM GB/s (% peak) at M=1; GEMM TFLOP/s (% MFMA) at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.WORKLOADS[cfg_id].dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "group": wl.WORKLOADS[cfg_id].group,
                   "matrices": [[m.name, m.N, m.K] for m in wl.WORKLOADS[cfg_id].matrices],
                   "bytes_per_step": step_bytes, "flops_per_step": step_flops},
        "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "tokens_per_s": round(M / (ms_per_step * 1e-3), 1),
        "roofline": roof,
        "grouped_step": grouped,
        "prefill": prefill,
        "formats": formats,
        "quality": quality,
        "awq_step": awq,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
