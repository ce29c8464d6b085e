// Offline quantise + pack, and the inverse view used by tests and tools.
//
// Quantiser: groupwise round-to-nearest. The rounding step q = round(w /
// scale) is the naive quantiser of "Quantization Is Not a Zip File" (section
// 3), applied per group of 32/64/128 weights ("Block locality", same section)
// or of 256 (the K-quant super-block size in that page's table of GGUF
// names). The zero-point format (asym4) follows the asymmetric example of the
// instagit comparison page ("Practical Code Examples"): range [min, max]
// including zero, (q - zero) * scale. The symmetric formats (sym4, sym8 =
// W8A16) follow its symmetric INT8 scheme ("INT8: Symmetric Integer
// Quantization"): scale max|w| / qmax, codes clamped to the signed range,
// stored offset by qmax + 1 so that they are unsigned. Every step is IEEE fp32 so that the integer
// codes are reproducible bit for bit: min/max are exact, the two divisions are
// correctly rounded (never a reciprocal multiply), rint rounds half to even,
// and the fp16 scale conversion is round-to-nearest-even with subnormals.
#include "decode_common.hpp"

namespace w4a16 {
namespace {

// One thread per (row n, run w of eight consecutive groups): it quantises
// the run's groups of row n in two passes over the fp32 weights (range, then
// codes), writes their codes, the eight scales (one 16-byte store: scales are
// [N][G8], G8 = K / GROUP rounded up to a multiple of 8, padded slots 0) and,
// for the zero-point format, the eight zero-points as one word of [N][G8 / 8].
template <int GROUP, int FMT>
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int N, int K,
                                                   uint32_t *__restrict__ qweight,
                                                   uint16_t *__restrict__ scales,
                                                   uint32_t *__restrict__ zeros) {
    using FT = FormatTraits<FMT>;
    constexpr int CPG = GROUP / kChunk;     // chunks per group
    constexpr int QMAX = FMT == kSym8 ? 127 : 7;   // symmetric: codes q + QMAX + 1, q in [-QMAX-1, QMAX]
    const int G = K / GROUP;
    const int W = (G + 7) / 8;              // runs of eight groups per row
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (n, run), run fastest
    if (tid >= (int64_t)W * N) return;
    const int n = (int)(tid / W);
    const int run = (int)(tid % W);
    const int64_t plane = (int64_t)N * K / 8;   // dwords of one 4-bit plane

    uint32_t sw[4] = {0u, 0u, 0u, 0u};   // the run's eight scales, two per word
    uint32_t zw = 0;                     // and zero-points, 4 bits each
    for (int e = 0; e < 8; ++e) {
        const int g = run * 8 + e;
        if (g >= G) break;   // padded slots stay 0
        const float4 *src = reinterpret_cast<const float4 *>(w + (int64_t)n * K + (int64_t)g * GROUP);
        // 1. range: [min(0, min w), max(0, max w)] or max|w|
        float lo = 0.0f, hi = 0.0f;
        for (int i = 0; i < GROUP / 4; ++i) {
            const float4 v = src[i];
            lo = fminf(fminf(fminf(lo, v.x), fminf(v.y, v.z)), v.w);
            hi = fmaxf(fmaxf(fmaxf(hi, v.x), fmaxf(v.y, v.z)), v.w);
        }
        const float amax = fmaxf(-lo, hi);
        // 2. scale, rounded once to fp16 (zero -> smallest positive fp16, 2^-24)
        const float s32 = FT::has_zeros ? (hi - lo) / 15.0f : amax / (float)QMAX;
        uint16_t sbits = f32_to_f16_bits(s32);
        if (sbits == 0) sbits = 1;
        const float sc = (float)__builtin_bit_cast(_Float16, sbits);
        int z = 0;
        if constexpr (FT::has_zeros) {
            z = (int)rintf(-lo / sc);
            z = z < 0 ? 0 : (z > 15 ? 15 : z);
        }
        // 3. codes, one dword (8 consecutive k) at a time
        for (int c = 0; c < CPG; ++c) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float4 a = src[c * 8 + d * 2], b = src[c * 8 + d * 2 + 1];
                const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t word = 0, word_hi = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    int q = (int)rintf(v[i] / sc);
                    if constexpr (FT::has_zeros) {
                        q += z;
                        q = q < 0 ? 0 : (q > 15 ? 15 : q);
                    } else {
                        q = q < -QMAX - 1 ? -QMAX - 1 : (q > QMAX ? QMAX : q);
                        q += QMAX + 1;
                    }
                    const int p = (i >> 1) + 4 * (i & 1);   // even k low half, odd k high half
                    word |= (uint32_t)(q & 0xF) << (4 * p);
                    word_hi |= (uint32_t)(q >> 4) << (4 * p);
                }
                const int64_t off = dword_offset(n, g * CPG + c, d, N, K);
                qweight[off] = word;
                if constexpr (FT::two_planes) qweight[plane + off] = word_hi;
            }
        }
        sw[e >> 1] |= (uint32_t)sbits << (16 * (e & 1));
        zw |= (uint32_t)z << (4 * e);
    }
    const int64_t G8 = (int64_t)W * 8;
    *reinterpret_cast<uint4 *>(scales + (int64_t)n * G8 + (int64_t)run * 8) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
    if constexpr (FT::has_zeros) zeros[(int64_t)n * W + run] = zw;
}

// K-quant-style super-blocks: one thread per (row n, 256-weight super-block
// u). Per 32-weight sub-block j: the range [min(0, min w), max(0, max w)]
// gives s_j = (hi - lo) / 15 and the minimum mn_j = 0 - lo; d and dmin are
// the largest s_j and mn_j over 63, rounded once to fp16 (0 -> 2^-24); the
// 6-bit sc_j, mq_j are rint(s_j / d) and rint(mn_j / dmin), clamped; codes
// are rint((w + M_j) / S_j), clamped to 0..15, with S_j = d sc_j and
// M_j = dmin mq_j (0 where S_j = 0). Writes the codes and the 16-byte record
// {d | dmin << 16, 48-bit sc field, 48-bit mq field} at [n][u].
__global__ __launch_bounds__(256) void pack_kq_kernel(const float *__restrict__ w, int N, int K,
                                                      uint32_t *__restrict__ qweight, uint4 *__restrict__ rec) {
    constexpr int SUB = 8;   // sub-blocks per super-block
    const int U = K / 256;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (u, n), n fastest
    if (tid >= (int64_t)U * N) return;
    const int n = (int)(tid % N), u = (int)(tid / N);
    const float4 *src = reinterpret_cast<const float4 *>(w + (int64_t)n * K + (int64_t)u * 256);
    float s[SUB], mn[SUB];
    float smax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < SUB; ++j) {
        float lo = 0.0f, hi = 0.0f;
        for (int i = 0; i < 8; ++i) {
            const float4 v = src[j * 8 + i];
            lo = fminf(fminf(fminf(lo, v.x), fminf(v.y, v.z)), v.w);
            hi = fmaxf(fmaxf(fmaxf(hi, v.x), fmaxf(v.y, v.z)), v.w);
        }
        s[j] = (hi - lo) / 15.0f;
        mn[j] = 0.0f - lo;
        smax = fmaxf(smax, s[j]);
        mmax = fmaxf(mmax, mn[j]);
    }
    uint16_t dbits = f32_to_f16_bits(smax / 63.0f), mbits = f32_to_f16_bits(mmax / 63.0f);
    if (dbits == 0) dbits = 1;
    if (mbits == 0) mbits = 1;
    const float d = (float)__builtin_bit_cast(_Float16, dbits), dm = (float)__builtin_bit_cast(_Float16, mbits);
    uint64_t scf = 0, mqf = 0;
    for (int j = 0; j < SUB; ++j) {
        int sc = (int)rintf(s[j] / d), mq = (int)rintf(mn[j] / dm);
        sc = sc < 0 ? 0 : (sc > 63 ? 63 : sc);
        mq = mq < 0 ? 0 : (mq > 63 ? 63 : mq);
        scf |= (uint64_t)sc << (6 * j);
        mqf |= (uint64_t)mq << (6 * j);
        const float S = d * (float)sc, M = dm * (float)mq;
        for (int dd = 0; dd < 4; ++dd) {
            const float4 a = src[j * 8 + dd * 2], b = src[j * 8 + dd * 2 + 1];
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int q = 0;
                if (S > 0.0f) {
                    q = (int)rintf((v[i] + M) / S);
                    q = q < 0 ? 0 : (q > 15 ? 15 : q);
                }
                word |= (uint32_t)q << (4 * ((i >> 1) + 4 * (i & 1)));   // even k low half, odd k high half
            }
            qweight[dword_offset(n, u * 8 + j, dd, N, K)] = word;
        }
    }
    rec[(int64_t)n * U + u] = make_uint4((uint32_t)dbits | ((uint32_t)mbits << 16), (uint32_t)scf,
                                         (uint32_t)(scf >> 32) | ((uint32_t)(mqf & 0xFFFFu) << 16),
                                         (uint32_t)(mqf >> 16));
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint32_t *__restrict__ qweight,
                                                           int N, int K, int planes,
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
    const uint32_t word_hi = planes == 2 ? qweight[(int64_t)N * KD + dword] : 0u;   // 8-bit codes: high nibbles
    uint8_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = 4 * ((i >> 1) + 4 * (i & 1));
        out[i] = ((word >> p) & 0xF) | (((word_hi >> p) & 0xF) << 4);
    }
    uint2 packed;
    packed.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
    packed.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
    *reinterpret_cast<uint2 *>(codes + (int64_t)n * K + 8 * kd) = packed;
}

// Metadata [N][G8] / [N][G8 / 8] -> canonical [G][N] scale bits and
// zero-points. fixed_zero: 0 when the zero-points are read from `zeros`, else
// the symmetric formats' fixed zero (8 or 128), written for every group.
__global__ __launch_bounds__(256) void unpack_meta_kernel(const uint16_t *__restrict__ scales,
                                                          const uint32_t *__restrict__ zeros,
                                                          int N, int G, int fixed_zero, uint16_t *__restrict__ s_out,
                                                          uint8_t *__restrict__ z_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // canonical (g, n)
    if (i >= (int64_t)G * N) return;
    const int g = (int)(i / N), n = (int)(i % N);
    const int64_t G8 = (int64_t)(G + 7) / 8 * 8;
    s_out[i] = scales[(int64_t)n * G8 + g];
    if (fixed_zero) {
        z_out[i] = (uint8_t)fixed_zero;
        return;
    }
    z_out[i] = (zeros[(int64_t)n * (G8 / 8) + g / 8] >> (4 * (g % 8))) & 0xF;
}

template <int FMT>
hipError_t launch_pack_fmt(const float *w, int N, int K, int group, uint32_t *q, uint16_t *s, uint32_t *z,
                           hipStream_t stream) {
    const int64_t total = ceil_div(K / group, 8) * N;   // (row, run of eight groups)
    const dim3 block(256);
    const dim3 grid((unsigned)ceil_div(total, 256));
    switch (group) {
        case 32: hipLaunchKernelGGL((pack_kernel<32, FMT>), grid, block, 0, stream, w, N, K, q, s, z); break;
        case 64: hipLaunchKernelGGL((pack_kernel<64, FMT>), grid, block, 0, stream, w, N, K, q, s, z); break;
        case 128: hipLaunchKernelGGL((pack_kernel<128, FMT>), grid, block, 0, stream, w, N, K, q, s, z); break;
        default: hipLaunchKernelGGL((pack_kernel<256, FMT>), grid, block, 0, stream, w, N, K, q, s, z); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const float *w, int N, int K, int group, int fmt, void *qweight, void *scales,
                       void *zeros, hipStream_t stream) {
    auto *q = reinterpret_cast<uint32_t *>(qweight);
    auto *s = reinterpret_cast<uint16_t *>(scales);
    auto *z = reinterpret_cast<uint32_t *>(zeros);
    if (fmt == kKq4) {
        const int64_t total = (int64_t)(K / 256) * N;
        hipLaunchKernelGGL(pack_kq_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream, w, N, K, q,
                           reinterpret_cast<uint4 *>(scales));
        return hipGetLastError();
    }
    switch (fmt) {
        case kSym4: return launch_pack_fmt<kSym4>(w, N, K, group, q, s, z, stream);
        case kSym8: return launch_pack_fmt<kSym8>(w, N, K, group, q, s, z, stream);
        default: return launch_pack_fmt<kAsym4>(w, N, K, group, q, s, z, stream);
    }
}

hipError_t launch_unpack(const void *qweight, const void *scales, const void *zeros, int N, int K,
                         int group, int fmt, uint8_t *codes, uint16_t *scales_out, uint8_t *zeros_out,
                         hipStream_t stream) {
    const int64_t nd = (int64_t)N * (K / 8);
    hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)ceil_div(nd, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(qweight), N, K, fmt == kSym8 ? 2 : 1, codes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fmt == kKq4) return e;   // kq4: its records are already in canonical order
    const int G = K / group;
    const int fz = fmt == kSym8 ? 128 : (fmt == kSym4 ? 8 : 0);
    const dim3 grid((unsigned)ceil_div((int64_t)G * N, 256));
    hipLaunchKernelGGL(unpack_meta_kernel, grid, dim3(256), 0, stream, reinterpret_cast<const uint16_t *>(scales),
                       reinterpret_cast<const uint32_t *>(zeros), N, G, fz, scales_out, zeros_out);
    return hipGetLastError();
}

}  // namespace w4a16
