"""Seeded synthetic inputs for the W4A16 linear layer.

This module is shared by the tests, the benchmark and the oracle's callers. It
draws random numbers and formats them (fp32 weights in the PyTorch ``Linear``
orientation [N][K], 16-bit activations as raw bit patterns [M][K]); it holds no
part of the quantise / pack / dequantise / multiply arithmetic.

Workloads (shapes from the decode and prefill cases of a 13B-class model with
hidden size 5120, as sized in "Weight-Only Quantization Explained", section
"The memory arithmetic"; the 70B-class down projection follows the 70B sizing
of "Quantization Is Not a Zip File", section 2):

  id  name               M            K      N      group  weights                      x
  1   gemv_4096          1            4096   4096   128    N(0, 0.02)                   fp16 N(0,1)
  2   decode_13b_layer   1            7 matrices (q,k,v,o 5120x5120; up, gate
                                      K=5120,N=13824; down K=13824,N=5120)   128
                                                          N(0, 0.02)                   fp16 N(0,1)
  3   fused_qkv          2,4,8,16     5120   15360  128    N(0, 0.02), 51 input
                                                          channels (1 %) scaled x20    fp16 N(0,1)
  4   prefill            2048         5120   13824  128    N(0, 0.02)                   bf16 N(0,1)
  5   ffn_down_70b       1, 8         28672  8192   32     Student-t(4) x 0.02          fp16 N(0,1)

Seeds: ``numpy.random.default_rng([config_id, matrix_id, role])`` with role 0
for weights and role 1 for activations (M appended for activations).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int
    K: int


@dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    ms: tuple
    group: int
    dtype: str
    matrices: tuple
    weight_dist: str = "normal"      # "normal" | "student_t4"
    outlier_channels: float = 0.0    # fraction of input channels scaled x20
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "gemv_4096", (1,), 128, F16, (Matrix("w", 4096, 4096),)),
    2: Workload(2, "decode_13b_layer", (1,), 128, F16, (
        Matrix("q", 5120, 5120), Matrix("k", 5120, 5120), Matrix("v", 5120, 5120),
        Matrix("o", 5120, 5120), Matrix("up", 13824, 5120), Matrix("gate", 13824, 5120),
        Matrix("down", 5120, 13824))),
    3: Workload(3, "fused_qkv", (2, 4, 8, 16), 128, F16, (Matrix("qkv", 15360, 5120),),
                outlier_channels=0.01),
    4: Workload(4, "prefill", (2048,), 128, BF16, (Matrix("up", 13824, 5120),)),
    5: Workload(5, "ffn_down_70b", (1, 8), 32, F16, (Matrix("down", 8192, 28672),),
                weight_dist="student_t4"),
}


def rng_for(config_id: int, matrix_id: int, role: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([config_id, matrix_id, role, *extra])


def weights(config_id: int, matrix_id: int) -> np.ndarray:
    """fp32 weights [N][K] for one matrix of a workload (seeded)."""
    wl = WORKLOADS[config_id]
    mat = wl.matrices[matrix_id]
    rng = rng_for(config_id, matrix_id, 0)
    if wl.weight_dist == "normal":
        w = rng.standard_normal((mat.N, mat.K), dtype=np.float32)
        w *= np.float32(0.02)
    elif wl.weight_dist == "student_t4":
        w = (rng.standard_t(4, size=(mat.N, mat.K)) * 0.02).astype(np.float32)
    else:
        raise ValueError(wl.weight_dist)
    if wl.outlier_channels:
        n_out = int(round(wl.outlier_channels * mat.K))
        cols = rng.choice(mat.K, size=n_out, replace=False)
        w[:, cols] *= np.float32(20.0)
    return w


def to_16bit(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 activations once to fp16 or bf16 (RNE); return the raw uint16 bits."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def activations(config_id: int, matrix_id: int, M: int) -> np.ndarray:
    """16-bit activations [M][K] (raw bits, dtype per workload), N(0,1) rounded once."""
    wl = WORKLOADS[config_id]
    mat = wl.matrices[matrix_id]
    rng = rng_for(config_id, matrix_id, 1, M)
    x = rng.standard_normal((M, mat.K), dtype=np.float32)
    return to_16bit(x, wl.dtype)


def random_weights(seed: int, N: int, K: int, scale: float = 0.02) -> np.ndarray:
    """Generic seeded fp32 N(0, scale) weights [N][K] for small test shapes."""
    rng = np.random.default_rng([seed, 0])
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(scale)
    return w


def random_activations(seed: int, M: int, K: int, dtype: str = F16) -> np.ndarray:
    """Generic seeded N(0,1) activations [M][K] as 16-bit bits."""
    rng = np.random.default_rng([seed, 1, M])
    return to_16bit(rng.standard_normal((M, K), dtype=np.float32), dtype)
