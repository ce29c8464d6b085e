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

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

__device__ inline v4u_t ld_nt(const v4u_t *p) { return __builtin_nontemporal_load(p); }

// Workgroup g reads the contiguous 16-byte words [g * per_wg, (g + 1) * per_wg)
// of the n16 words: thread t takes words t, t + 256, ..., four loads in flight
// (each load instruction of a wave reads one contiguous KiB). The words are
// folded into one value that is stored only if it equals a constant, so the
// loads cannot be dropped and (in practice) nothing is written.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u_t *__restrict__ src, size_t n16, size_t per_wg,
                                                          uint32_t *__restrict__ sink) {
    const size_t begin = (size_t)blockIdx.x * per_wg;
    const size_t end = begin + per_wg < n16 ? begin + per_wg : n16;
    size_t i = begin + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * 256 < end; i += 4 * 256) {
        const v4u_t a = ld_nt(src + i), b = ld_nt(src + i + 256), c = ld_nt(src + i + 512), d = ld_nt(src + i + 768);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < end; i += 256) {
        const v4u_t a = ld_nt(src + i);
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

int copy_grid() {
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
    const size_t n16 = bytes / 16;
    // default: 16 KiB per workgroup (four loads per thread, one pass)
    const size_t per_wg = workgroups > 0 ? (n16 + workgroups - 1) / workgroups : 1024;
    const size_t grid = (n16 + per_wg - 1) / per_wg;
    if (grid > 0x7FFFFFFFull) return W4A16_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const v4u_t *>(src), n16, per_wg, sink);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_measure_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
        return W4A16_ERR_INVALID_ARG;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return W4A16_ERR_INVALID_ARG;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)copy_grid()), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4 *>(src),
                       reinterpret_cast<uint4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

}  // extern "C"
