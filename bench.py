#!/usr/bin/env python3
"""Benchmark of the gfx950 W4A16 linear layer.

Default workload: the decode layer set of a 13B-class model at M = 1 (q, k, v,
o: 5120x5120; up, gate: K=5120, N=13824; down: K=13824, N=5120; group 128,
fp16 activations). One step = one token through all seven W4A16 linear layers
(seven w4a16_linear calls, which dispatch to the GEMV kernel at M = 1). Inputs
are synthetic and seeded; the packed weights are rotated over enough copies to
exceed the 256 MB last-level cache, so every step streams its weights from HBM.

Prints one JSON line. `value` is achieved HBM GB/s over the step (algorithmic
bytes: packed weights + scales + zeros + activations read + outputs written,
divided by wall time per step). `roofline` gives the GEMV kernel's own rate
from HIP events around each launch, against the 8 TB/s HBM3E peak.
`cpu_baseline` times the CPU oracle (dequantise + fp64 product) on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_13b_layer",
                   choices=["decode_13b_layer", "gemv_4096", "fused_qkv", "prefill", "ffn_down_70b"])
    p.add_argument("--m", type=int, default=0, help="batch rows (default: the workload's first M)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain device copy of known size (for counter scaling)")
    return p.parse_args()


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "w4a16_weight_only_dequant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(M, N, K, group):
    G = K // group
    return N * K // 2 + 2 * G * N + G * N // 2 + 2 * M * K + 2 * M * N


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import w4a16_weight_only_dequant_amd as w4
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    assert w4.device_supported(0), "cuda:0 is not a gfx950"

    cfg_id = {"gemv_4096": 1, "decode_13b_layer": 2, "fused_qkv": 3, "prefill": 4, "ffn_down_70b": 5}[args.workload]
    wcfg = wl.WORKLOADS[cfg_id]
    M = args.m or wcfg.ms[0]
    group = wcfg.group
    dtype = wcfg.dtype
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16

    # ---- setup: pack every matrix once, then rotate copies past the MALL ----
    packed, xs, ys, mats = [], [], [], []
    for mi, mat in enumerate(wcfg.matrices):
        w = torch.from_numpy(wl.weights(cfg_id, mi)).to(dev)
        packed.append(w4.pack(w, group))
        del w
        xb = wl.activations(cfg_id, mi, M)
        xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(tdt))
        ys.append(torch.empty((M, mat.N), dtype=tdt, device=dev))
        mats.append(mat)
    torch.cuda.synchronize()
    set_bytes = sum(p.nbytes() for p in packed)
    copies = max(1, -(-3 * MALL_BYTES // set_bytes))
    sets = [packed]
    for _ in range(copies - 1):
        sets.append([w4.PackedWeight(p.qweight.clone(), p.scales.clone(), p.zeros.clone(), p.N, p.K, p.group)
                     for p in packed])
    ws = w4.Workspace(dev)
    step_bytes = sum(algorithmic_bytes(M, m.N, m.K, group) for m in mats)
    step_flops = sum(2 * M * m.N * m.K for m in mats)

    def step(i, events=None):
        s = sets[i % copies]
        for j, pw in enumerate(s):
            if events is not None:
                events[j][0].record()
            w4.linear(xs[j], pw, out=ys[j], workspace=ws)
            if events is not None:
                events[j][1].record()

    # eager warm-up (allocates the workspace), then HIP graphs: one graph per
    # weight copy holding one step, and one graph per matrix holding one launch
    # on every copy (for the per-kernel timing). Graph replay keeps the GPU fed
    # without per-launch host overhead.
    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream(device=dev)
    step_graphs, mat_graphs = [], []
    with torch.cuda.stream(cap):
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(c)
            step_graphs.append(g)
        for j, m in enumerate(mats):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for c in range(copies):
                    w4.linear(xs[j], sets[c][j], out=ys[j], workspace=ws)
            mat_graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step_graphs[i % copies].replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, bracketed by synchronisation ----
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step_graphs[i % copies].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---- per-kernel timing: HIP events on the launch stream around each
    # matrix's graph (one launch per weight copy, back to back) ----
    n_mat = len(mats)
    reps = max(1, args.steps // (copies * 4))
    per_mat_ms = np.zeros(n_mat)
    for j in range(n_mat):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        mat_graphs[j].replay()
        a0.record()
        for _ in range(reps):
            mat_graphs[j].replay()
        a1.record()
        torch.cuda.synchronize()
        per_mat_ms[j] = a0.elapsed_time(a1) / (reps * copies)
    kernel_ms_step = float(per_mat_ms.sum())

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (kernel_ms_step * 1e-3) / 1e9

    uses_gemv = M <= w4.gemv_max_m()
    bound = "hbm" if uses_gemv or M <= 64 else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        tf = step_flops / (kernel_ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    kernel_file = "gemv.hip" if uses_gemv else "gemm.hip"
    src_hash = kernel_source_hash([kernel_file, "w4a16_internal.hpp"])
    roof["kernel"] = "gemv_kernel" if uses_gemv else "gemm_kernel"
    roof["kernel_source_sha"] = src_hash
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{args.workload}_m{M}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("kernel_source_sha") == src_hash:
            roof["traffic"] = t.get("traffic_bytes_per_step")
    roof["units_per_launch"] = {m.name: {"weights": m.N * m.K, "bytes": algorithmic_bytes(M, m.N, m.K, group),
                                         "kernel_us": round(float(per_mat_ms[j]) * 1e3, 2)}
                                for j, m in enumerate(mats)}

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.uint8, device=dev)   # 256 MiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import w4a16_ref as ref
        cores = len(os.sched_getaffinity(0))
        done_bytes, t_cpu, names = 0, 0.0, []
        mi = 0
        while t_cpu < args.cpu_seconds and mi < 2 * n_mat:
            j = mi % n_mat
            codes, s_bits, zeros = ref.quantize_groupwise(wl.weights(cfg_id, j), group)   # offline, untimed
            xb = wl.activations(cfg_id, j, M)
            t1 = time.perf_counter()
            w_hat = ref.dequantize(codes, s_bits, zeros, group)
            ref.linear_ref(xb, dtype, w_hat)
            t_cpu += time.perf_counter() - t1
            done_bytes += algorithmic_bytes(M, mats[j].N, mats[j].K, group)
            names.append(mats[j].name)
            mi += 1
            del w_hat, codes
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"dequantise + fp64 product (numpy) for matrices {','.join(names)} at M={M}, "
                         f"{t_cpu:.1f} s; threads = host affinity count (BLAS), dequantise single-threaded"}

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
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "group": group,
                   "matrices": [[m.name, m.N, m.K] for m in mats],
                   "bytes_per_step": step_bytes, "flops_per_step": step_flops,
                   "weight_copies_rotated": copies},
        "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "tokens_per_s": round(M / (ms_per_step * 1e-3), 1),
        "tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
