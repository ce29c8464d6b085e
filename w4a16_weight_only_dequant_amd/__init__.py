"""MI355X (gfx950) W4A16 weight-only linear layer.

The compute lives in libw4a16.so (hand-written HIP kernels behind a C ABI,
include/w4a16.h); this package is its thin Python binding.
"""
from ._lib import (EXPORTED, FORMATS, LIB_PATH, PackedWeight, W4A16Error, Workspace, device_supported, init,  # noqa: F401
                   gemm, gemv, gemv_max_m, linear, linear_awq, linear_group, linear_kernel, linear_launch_shape,
                   linear_noalloc, linear_run, pack,
                   packed_bytes,
                   QUALITY_FIELDS, quant_error, raw, scale_activations, unpack, workspace_bytes)
