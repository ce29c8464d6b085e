"""Host-side checks of the benchmark script: the one-GPU contract and the byte
accounting it reports (no GPU needed)."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_per_format():
    from oracle import w4a16_ref as ref
    b = _bench()
    for N, K, g in ((5120, 5120, 128), (13824, 5120, 128), (8192, 28672, 32)):
        for fmt in ("asym4", "sym4", "sym8"):
            q, s, z = ref.packed_bytes(N, K, g, fmt)
            assert b.algorithmic_bytes(1, N, K, g, fmt) == q + s + z + 2 * K + 2 * N
    q, s, z = ref.packed_bytes(5120, 13824, 256, "kq4")
    assert b.algorithmic_bytes(4, 5120, 13824, 256, "kq4") == q + s + z + 2 * 4 * 13824 + 2 * 4 * 5120
    # the headline step: the 13B decode layer set at group 128, M = 1
    assert sum(b.algorithmic_bytes(1, N, K, 128) for N, K in
               [(5120, 5120)] * 4 + [(13824, 5120)] * 2 + [(5120, 13824)]) == 4 * 13639680 + 3 * 36809728


def test_stored_traffic_is_reported_only_for_the_counted_sources(monkeypatch):
    b = _bench()
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic_decode_13b_layer_m1.json")))
    same = t["kernel_source_sha"] == b.kernel_source_hash("gemv")
    assert b.stored_traffic("decode_13b_layer", 1, "gemv") == (t["traffic_bytes_per_launch_set"] if same else None)
    monkeypatch.setattr(b, "kernel_source_hash", lambda kind: "0" * 16)   # sources changed since the count
    assert b.stored_traffic("decode_13b_layer", 1, "gemv") is None
    assert b.stored_traffic("decode_13b_layer", 2, "gemv") is None            # no counter run for M = 2
