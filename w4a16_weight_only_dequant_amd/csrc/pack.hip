// Offline quantise + pack, and the inverse view used by tests and tools.
//
// Quantiser: groupwise asymmetric round-to-nearest. The rounding step
// q = round(w / scale) is the naive quantiser of "Quantization Is Not a Zip
// File" (section 3), applied per group of 32/64/128 weights ("Block
// locality", same section); the zero-point and (q - zero) * scale
// reconstruction follow the asymmetric example of the instagit comparison
// page ("Practical Code Examples"). Every step is IEEE fp32 so that the integer
// codes are reproducible bit for bit: min/max are exact, the two divisions are
// correctly rounded (never a reciprocal multiply), rint rounds half to even,
// and the fp16 scale conversion is round-to-nearest-even with subnormals.
#include "w4a16_internal.hpp"

namespace w4a16 {
namespace {

template <int GROUP>
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int N, int K,
                                                   uint4 *__restrict__ qweight,
                                                   uint16_t *__restrict__ scales,
                                                   uint32_t *__restrict__ zeros) {
    constexpr int CPG = GROUP / kChunk;
    const int G = K / GROUP;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (g, n), n fastest
    const bool active = t < (int64_t)G * N;
    const int n = active ? (int)(t % N) : 0;
    const int g = active ? (int)(t / N) : 0;

    float vals[GROUP];
    float lo = 0.0f, hi = 0.0f;   // the range always contains zero
    if (active) {
        const float4 *src = reinterpret_cast<const float4 *>(w + (int64_t)n * K + (int64_t)g * GROUP);
#pragma unroll
        for (int i = 0; i < GROUP / 4; ++i) {
            float4 v = src[i];
            vals[4 * i + 0] = v.x;
            vals[4 * i + 1] = v.y;
            vals[4 * i + 2] = v.z;
            vals[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < GROUP; ++i) {
            lo = fminf(lo, vals[i]);
            hi = fmaxf(hi, vals[i]);
        }
    }
    const float s32 = (hi - lo) / 15.0f;
    uint16_t sbits = f32_to_f16_bits(s32);
    if (sbits == 0) sbits = 1;                           // smallest positive fp16, 2^-24
    const float s = (float)__builtin_bit_cast(_Float16, sbits);
    int z = (int)rintf(-lo / s);
    z = z < 0 ? 0 : (z > 15 ? 15 : z);

    if (active) {
        const int rb = n / kRowBlock;
        const int r = n % kRowBlock;
        const int rows_b = min(kRowBlock, N - rb * kRowBlock);
        uint4 *dst = qweight + (int64_t)rb * 2 * K + r;   // 64 rows * K/2 bytes / 16 = 2K records
#pragma unroll
        for (int c = 0; c < CPG; ++c) {
            uint32_t dw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t word = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    int q = (int)rintf(vals[c * 32 + j * 8 + i] / s) + z;
                    q = q < 0 ? 0 : (q > 15 ? 15 : q);
                    const int p = (i >> 1) + 4 * (i & 1);   // even k low half, odd k high half
                    word |= (uint32_t)q << (4 * p);
                }
                dw[j] = word;
            }
            const int chunk = g * CPG + c;
            dst[(int64_t)chunk * rows_b] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
        }
        scales[(int64_t)g * N + n] = sbits;
    }
    // zeros: 8 consecutive n share one word; N % 8 == 0 and t runs n fastest,
    // so each aligned octet of lanes is complete and belongs to one word.
    uint32_t zw = active ? ((uint32_t)z << (4 * (n & 7))) : 0u;
    zw |= __shfl_xor(zw, 1, 64);
    zw |= __shfl_xor(zw, 2, 64);
    zw |= __shfl_xor(zw, 4, 64);
    if (active && (n & 7) == 0) zeros[(int64_t)g * (N / 8) + n / 8] = zw;
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint32_t *__restrict__ qweight,
                                                           int N, int K,
                                                           uint8_t *__restrict__ codes) {
    // one thread per (n, 8-weight dword) in canonical order
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int KD = K / 8;
    if (t >= (int64_t)N * KD) return;
    const int n = (int)(t / KD);
    const int kd = (int)(t % KD);
    const int rb = n / kRowBlock, r = n % kRowBlock;
    const int rows_b = min(kRowBlock, N - rb * kRowBlock);
    const int c = kd / 4, j = kd % 4;
    const int64_t dword = ((int64_t)rb * 2 * K + (int64_t)c * rows_b + r) * 4 + j;
    const uint32_t word = qweight[dword];
    uint8_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (word >> (4 * ((i >> 1) + 4 * (i & 1)))) & 0xF;
    uint2 packed;
    packed.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
    packed.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
    *reinterpret_cast<uint2 *>(codes + (int64_t)n * K + 8 * kd) = packed;
}

__global__ __launch_bounds__(256) void unpack_meta_kernel(const uint16_t *__restrict__ scales,
                                                          const uint32_t *__restrict__ zeros,
                                                          int64_t GN, uint16_t *__restrict__ s_out,
                                                          uint8_t *__restrict__ z_out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= GN) return;
    s_out[t] = scales[t];
    z_out[t] = (zeros[t / 8] >> (4 * (t & 7))) & 0xF;
}

}  // namespace

hipError_t launch_pack(const float *w, int N, int K, int group, void *qweight, void *scales,
                       void *zeros, hipStream_t stream) {
    const int64_t total = (int64_t)(K / group) * N;
    const dim3 block(256);
    const dim3 grid((unsigned)ceil_div(total, 256));
    auto *q = reinterpret_cast<uint4 *>(qweight);
    auto *s = reinterpret_cast<uint16_t *>(scales);
    auto *z = reinterpret_cast<uint32_t *>(zeros);
    switch (group) {
        case 32: hipLaunchKernelGGL(pack_kernel<32>, grid, block, 0, stream, w, N, K, q, s, z); break;
        case 64: hipLaunchKernelGGL(pack_kernel<64>, grid, block, 0, stream, w, N, K, q, s, z); break;
        default: hipLaunchKernelGGL(pack_kernel<128>, grid, block, 0, stream, w, N, K, q, s, z); break;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const void *qweight, const void *scales, const void *zeros, int N, int K,
                         int group, uint8_t *codes, uint16_t *scales_out, uint8_t *zeros_out,
                         hipStream_t stream) {
    const int64_t nd = (int64_t)N * (K / 8);
    hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)ceil_div(nd, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(qweight), N, K, codes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t gn = (int64_t)(K / group) * N;
    hipLaunchKernelGGL(unpack_meta_kernel, dim3((unsigned)ceil_div(gn, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t *>(scales),
                       reinterpret_cast<const uint32_t *>(zeros), gn, scales_out, zeros_out);
    return hipGetLastError();
}

}  // namespace w4a16
