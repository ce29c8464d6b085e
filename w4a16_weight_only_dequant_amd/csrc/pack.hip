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
#include "decode_common.hpp"

namespace w4a16 {
namespace {

// One thread per (row n, column t of 128 weights): quantises the column's
// 128/GROUP groups of row n, writes their codes, scales and zero-points.
template <int GROUP>
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int N, int K,
                                                   uint32_t *__restrict__ qweight,
                                                   uint16_t *__restrict__ scales,
                                                   uint32_t *__restrict__ zeros) {
    constexpr int CPG = GROUP / kChunk;     // chunks per group
    constexpr int GPC = kColumn / GROUP;    // groups per column
    const int C = K / kChunk;
    const int T = (C + kColChunks - 1) / kColChunks;
    const int G = K / GROUP;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (t, n), n fastest
    const bool active = tid < (int64_t)T * N;
    const int n = active ? (int)(tid % N) : 0;
    const int t = active ? (int)(tid / N) : 0;

    uint32_t znib = 0;   // the GPC zero-points of (t, n), 4 bits each
#pragma unroll
    for (int e = 0; e < GPC; ++e) {
        const int g = t * GPC + e;
        const bool real = active && g < G;
        float vals[GROUP];
        float lo = 0.0f, hi = 0.0f;   // the range always contains zero
        if (real) {
            const float4 *src = reinterpret_cast<const float4 *>(w + (int64_t)n * K + (int64_t)g * GROUP);
#pragma unroll
            for (int i = 0; i < GROUP / 4; ++i) {
                const float4 v = src[i];
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
        const float sc = (float)__builtin_bit_cast(_Float16, sbits);
        int z = (int)rintf(-lo / sc);
        z = z < 0 ? 0 : (z > 15 ? 15 : z);
        if (real) {
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t word = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        int q = (int)rintf(vals[c * 32 + d * 8 + i] / sc) + z;
                        q = q < 0 ? 0 : (q > 15 ? 15 : q);
                        const int p = (i >> 1) + 4 * (i & 1);   // even k low half, odd k high half
                        word |= (uint32_t)q << (4 * p);
                    }
                    qweight[dword_offset(n, g * CPG + c, d, N, K)] = word;
                }
            }
        }
        if (active) scales[((int64_t)t * N + n) * GPC + e] = real ? sbits : (uint16_t)0;
        znib |= (real ? (uint32_t)z : 0u) << (4 * e);
    }
    // zeros: word (t, i) holds the nibbles of rows 8/GPC*i .. 8/GPC*i + 8/GPC-1;
    // N % 8 == 0 and tid runs n fastest, so those rows sit in neighbouring lanes
    constexpr int RPW = 8 / GPC;    // rows per zero word
    uint32_t zw = active ? znib << (4 * GPC * (n % RPW)) : 0u;
#pragma unroll
    for (int off = 1; off < RPW; off <<= 1) zw |= __shfl_xor(zw, off, 64);
    if (active && n % RPW == 0) zeros[(int64_t)t * (N / RPW) + n / RPW] = zw;
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
    const int c = kd / 4, j = kd % 4;
    const int64_t dword = dword_offset(n, c, j, N, K);
    const uint32_t word = qweight[dword];
    uint8_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (word >> (4 * ((i >> 1) + 4 * (i & 1)))) & 0xF;
    uint2 packed;
    packed.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
    packed.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
    *reinterpret_cast<uint2 *>(codes + (int64_t)n * K + 8 * kd) = packed;
}

template <int GROUP>
__global__ __launch_bounds__(256) void unpack_meta_kernel(const uint16_t *__restrict__ scales,
                                                          const uint32_t *__restrict__ zeros,
                                                          int N, int G, uint16_t *__restrict__ s_out,
                                                          uint8_t *__restrict__ z_out) {
    constexpr int GPC = kColumn / GROUP;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // canonical (g, n)
    if (i >= (int64_t)G * N) return;
    const int g = (int)(i / N), n = (int)(i % N);
    const int t = g / GPC, e = g % GPC;
    s_out[i] = scales[((int64_t)t * N + n) * GPC + e];
    const int64_t nib = (int64_t)t * N * GPC + (int64_t)n * GPC + e;
    z_out[i] = (zeros[nib / 8] >> (4 * (nib % 8))) & 0xF;
}

}  // namespace

hipError_t launch_pack(const float *w, int N, int K, int group, void *qweight, void *scales,
                       void *zeros, hipStream_t stream) {
    const int64_t total = ceil_div(K / kChunk, kColChunks) * N;   // (column, row) pairs
    const dim3 block(256);
    const dim3 grid((unsigned)ceil_div(total, 256));
    auto *q = reinterpret_cast<uint32_t *>(qweight);
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
    const int G = K / group;
    const dim3 grid((unsigned)ceil_div((int64_t)G * N, 256));
    auto *sc = reinterpret_cast<const uint16_t *>(scales);
    auto *zp = reinterpret_cast<const uint32_t *>(zeros);
    switch (group) {
        case 32: hipLaunchKernelGGL(unpack_meta_kernel<32>, grid, dim3(256), 0, stream, sc, zp, N, G, scales_out, zeros_out); break;
        case 64: hipLaunchKernelGGL(unpack_meta_kernel<64>, grid, dim3(256), 0, stream, sc, zp, N, G, scales_out, zeros_out); break;
        default: hipLaunchKernelGGL(unpack_meta_kernel<128>, grid, dim3(256), 0, stream, sc, zp, N, G, scales_out, zeros_out); break;
    }
    return hipGetLastError();
}

}  // namespace w4a16
