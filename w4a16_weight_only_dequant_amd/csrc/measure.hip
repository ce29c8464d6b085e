// Measurement kernels of the benchmark: a plain streaming read with 16-byte
// loads (the achievable HBM read rate, reported beside the product kernels as
// a ceiling, not used as their denominator) and a plain 16-byte copy (a
// kernel of known traffic that scales the HBM byte counters of a profiler
// run). Neither is on the product path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a16.h"
#include "w4a16_internal.hpp"

namespace {

// Grid-stride over n16 16-byte words, four loads in flight per thread. The
// words are folded into one value that is stored only if it equals a
// constant, so the loads cannot be dropped and (in practice) nothing is
// written.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) atomicOr(sink, acc);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                   size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int default_grid(int32_t workgroups) {
    if (workgroups > 0) return workgroups;
    const int cus = w4a16::device_cu_count();
    return 8 * (cus > 0 ? cus : 256);
}

}  // namespace

extern "C" {

w4a16_status w4a16_measure_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups,
                                       void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || workgroups < 0 ||
        workgroups > (1 << 20))
        return W4A16_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)default_grid(workgroups)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4 *>(src), bytes / 16,
                       sink);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_measure_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
        return W4A16_ERR_INVALID_ARG;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return W4A16_ERR_INVALID_ARG;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)default_grid(0)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4 *>(src),
                       reinterpret_cast<uint4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

}  // extern "C"
