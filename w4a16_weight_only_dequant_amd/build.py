"""Build the gfx950 HIP library libw4a16.so in-tree (hipcc, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libw4a16.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "pack.hip", "quality.hip", "measure.hip",
           "decode.hip", "decode_sym4.hip", "decode_sym8.hip", "decode_kq4.hip",
           "gemm.hip", "gemm_sym4.hip", "gemm_sym8.hip", "gemm_kq4.hip",
           "prefill.hip", "prefill_sym4.hip", "prefill_sym8.hip", "prefill_kq4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Werror", "-Wno-unused-function",
    # correctly rounded fp32 division (the quantiser's codes depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) for {cmd[-1]}")
    return r


def build(verbose: bool = False, jobs: int = 8, out: str = OUT, extra_flags=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every HIP source for gfx950 and link libw4a16.so (next to this file by default)."""
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra_flags, "-c", "-o", obj, os.path.join(CSRC, src)])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = out + ".tmp"
    # export the C ABI only (w4a16_*); internal C++ symbols stay local
    exports = os.path.join(CSRC, "exports.map")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", f"-Wl,--version-script={exports}", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
