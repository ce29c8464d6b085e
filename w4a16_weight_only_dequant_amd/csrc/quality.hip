// Quantisation quality report and AWQ's activation scaling.
//
// Quality report: the four figures of the error-analysis routine the instagit
// comparison page lists ("Implementation Architecture"): mean squared error,
// signal-to-noise ratio in dB, cosine similarity and largest error between the
// fp32 weights and the weights the packed data rebuilds, w_hat = s * (q - z),
// over the whole matrix, in fp64. One workgroup per (16-row block, slice of
// K's 128-weight columns) streams its share of the fp32 weights and the packed
// codes once and writes five partial sums; one workgroup then folds the
// partials in a fixed order (deterministic) and derives the four figures.
//
// AWQ's run-time half: the activations are multiplied by per-input-channel
// fp32 factors (the reciprocals of the factors the weights were scaled up by
// before quantisation; instagit page, "AWQ: Activation-Aware Weight
// Quantization") and rounded once to the activation type. The decode GEMV
// folds this into its activation staging; this elementwise kernel serves the
// other paths.
#include <math.h>

#include <algorithm>

#include "decode_common.hpp"

namespace w4a16 {
namespace {

constexpr int kQeThreads = 256;

struct Sums5 {
    double d2, w2, h2, wh, mx;
};

// Fixed-order reduction of the workgroup's sums into every lane of wave 0:
// a butterfly inside each wave, then wave 0 adds the waves' totals in order.
__device__ inline void block_reduce(Sums5 &v, double (*sh)[kQeThreads / 64]) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        v.d2 += __shfl_xor(v.d2, o);
        v.w2 += __shfl_xor(v.w2, o);
        v.h2 += __shfl_xor(v.h2, o);
        v.wh += __shfl_xor(v.wh, o);
        v.mx = fmax(v.mx, __shfl_xor(v.mx, o));
    }
    const int wave = threadIdx.x / 64;
    if (threadIdx.x % 64 == 0) {
        sh[0][wave] = v.d2;
        sh[1][wave] = v.w2;
        sh[2][wave] = v.h2;
        sh[3][wave] = v.wh;
        sh[4][wave] = v.mx;
    }
    __syncthreads();
    v = Sums5{sh[0][0], sh[1][0], sh[2][0], sh[3][0], sh[4][0]};
#pragma unroll
    for (int i = 1; i < kQeThreads / 64; ++i) {
        v.d2 += sh[0][i];
        v.w2 += sh[1][i];
        v.h2 += sh[2][i];
        v.wh += sh[3][i];
        v.mx = fmax(v.mx, sh[4][i]);
    }
}

// Slices of K per row block: enough workgroups to fill the chip (a row block
// alone is too little work for the 5120-row matrices), never less than one
// 128-weight column each.
#ifndef W4A16_QE_TARGET_WGS
#define W4A16_QE_TARGET_WGS 2048
#endif
constexpr int kQeTargetWgs = W4A16_QE_TARGET_WGS;
inline int qe_slices(int N, int K) {
    const int64_t blocks = ceil_div(N, kRowBlock), cols = ceil_div(K, kColumn);
    return (int)std::max<int64_t>(1, std::min<int64_t>(cols, ceil_div(kQeTargetWgs, blocks)));
}

// Workgroup g = b * slices + s takes row block b and the columns
// [s * cols / slices, (s + 1) * cols / slices): thread i walks its (row,
// 8-weight dword) pairs, rebuilds the eight weights from the packed layout
// and accumulates against the fp32 originals.
__global__ __launch_bounds__(kQeThreads) void quant_error_partial_kernel(
    const float *__restrict__ w, const uint32_t *__restrict__ qw, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ zeros, int N, int K, int group, int fmt, int slices,
    double *__restrict__ partial) {
    __shared__ double sh[5][kQeThreads / 64];
    const int b = blockIdx.x / slices, sl = blockIdx.x % slices;
    const int rows = min(kRowBlock, N - b * kRowBlock);
    const int cols = (K + kColumn - 1) / kColumn;
    const int kd0 = (int)((int64_t)sl * cols / slices) * (kColumn / 8);
    const int kd1 = min(K / 8, (int)((int64_t)(sl + 1) * cols / slices) * (kColumn / 8));
    const int KD = kd1 - kd0;
    const int G8 = meta_slots(K, group);                      // metadata slots per row
    const int64_t plane = (int64_t)N * K / 8;                 // dwords of one 4-bit plane
    const uint32_t fixed_zero = fmt == kSym8 ? 128u : (fmt == kKq4 ? 0u : 8u);
    Sums5 v{0.0, 0.0, 0.0, 0.0, 0.0};
    for (int i = threadIdx.x; i < rows * KD; i += kQeThreads) {
        const int r = i / KD, kd = kd0 + i % KD;
        const int n = b * kRowBlock + r;
        const int k0 = kd * 8;
        const int64_t off = dword_offset(n, kd / 4, kd % 4, N, K);
        const uint32_t lo = qw[off];
        const uint32_t hi = fmt == kSym8 ? qw[plane + off] : 0u;
        double s, mn = 0.0;
        uint32_t z = fixed_zero;
        if (fmt == kKq4) {   // sub-block (k0 % 256) / 32 of the record [n][k0 / 256]
            const uint4 rec = reinterpret_cast<const uint4 *>(scales)[(int64_t)n * (K / 256) + k0 / 256];
            const KqParams P = kq_params(rec, (k0 % 256) / kChunk);
            s = (double)P.S;
            mn = (double)P.M;
            z = 0;
        } else {
            const int g = k0 / group;
            s = (double)(float)__builtin_bit_cast(_Float16, scales[(int64_t)n * G8 + g]);
            if (fmt == kAsym4) z = (zeros[(int64_t)n * (G8 / 8) + g / 8] >> (4 * (g % 8))) & 0xFu;
        }
        const float4 wa = *reinterpret_cast<const float4 *>(w + (int64_t)n * K + k0);
        const float4 wb = *reinterpret_cast<const float4 *>(w + (int64_t)n * K + k0 + 4);
        const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = 4 * ((j >> 1) + 4 * (j & 1));   // even k in the low half-word
            const uint32_t q = ((lo >> p) & 0xFu) | (((hi >> p) & 0xFu) << 4);
            const double h = s * (double)((int)q - (int)z) - mn;
            const double x = (double)wv[j];
            const double d = x - h;
            v.d2 = fma(d, d, v.d2);
            v.w2 = fma(x, x, v.w2);
            v.h2 = fma(h, h, v.h2);
            v.wh = fma(x, h, v.wh);
            v.mx = fmax(v.mx, fabs(d));
        }
    }
    block_reduce(v, sh);
    if (threadIdx.x == 0) {
        double *o = partial + (int64_t)blockIdx.x * 5;
        o[0] = v.d2;
        o[1] = v.w2;
        o[2] = v.h2;
        o[3] = v.wh;
        o[4] = v.mx;
    }
}

// out = {MSE, SNR dB, cosine, max error, sum d^2, sum w^2, sum w_hat^2, sum w w_hat}
__global__ __launch_bounds__(kQeThreads) void quant_error_final_kernel(const double *__restrict__ partial,
                                                                       int blocks, double count,
                                                                       double *__restrict__ out) {
    __shared__ double sh[5][kQeThreads / 64];
    Sums5 v{0.0, 0.0, 0.0, 0.0, 0.0};
    for (int b = threadIdx.x; b < blocks; b += kQeThreads) {
        const double *p = partial + (int64_t)b * 5;
        v.d2 += p[0];
        v.w2 += p[1];
        v.h2 += p[2];
        v.wh += p[3];
        v.mx = fmax(v.mx, p[4]);
    }
    block_reduce(v, sh);
    if (threadIdx.x == 0) {
        const double inf = __builtin_huge_val();
        const double snr = v.d2 == 0.0 ? inf : (v.w2 > 0.0 ? 10.0 * log10(v.w2 / v.d2) : -inf);
        double cs;
        if (v.w2 == 0.0 && v.h2 == 0.0) cs = 1.0;
        else if (v.w2 == 0.0 || v.h2 == 0.0) cs = 0.0;
        else cs = v.wh / sqrt(v.w2 * v.h2);
        out[0] = v.d2 / count;
        out[1] = snr;
        out[2] = cs;
        out[3] = v.mx;
        out[4] = v.d2;
        out[5] = v.w2;
        out[6] = v.h2;
        out[7] = v.wh;
    }
}

// One thread per eight activations (16 bytes).
template <bool BF>
__global__ __launch_bounds__(256) void scale_activations_kernel(const uint4 *__restrict__ x,
                                                                const float4 *__restrict__ m, uint4 *__restrict__ out,
                                                                int64_t units, int units_per_row) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= units) return;
    const int u = (int)(i % units_per_row);
    const uint4 v = x[i];
    const float4 a = m[2 * u], b = m[2 * u + 1];
    const float mm[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float lo, hi;
        if constexpr (BF) {
            lo = __builtin_bit_cast(float, in[j] << 16);
            hi = __builtin_bit_cast(float, in[j] & 0xFFFF0000u);
        } else {
            const half2_t h = __builtin_bit_cast(half2_t, in[j]);
            lo = (float)h.x;
            hi = (float)h.y;
        }
        const float2_t p = {lo * mm[2 * j], hi * mm[2 * j + 1]};
        if constexpr (BF)
            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf162_t));
        else
            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, half2_t));
    }
    out[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

size_t quant_error_partial_bytes(int N, int K) {
    return (size_t)ceil_div(N, kRowBlock) * qe_slices(N, K) * 5 * sizeof(double);
}

hipError_t launch_quant_error(const float *w, const void *qweight, const void *scales, const void *zeros, int N,
                              int K, int group, int fmt, double *out, double *partial, hipStream_t stream) {
    const int slices = qe_slices(N, K);
    const int blocks = (int)ceil_div(N, kRowBlock) * slices;
    hipLaunchKernelGGL(quant_error_partial_kernel, dim3(blocks), dim3(kQeThreads), 0, stream, w,
                       reinterpret_cast<const uint32_t *>(qweight), reinterpret_cast<const uint16_t *>(scales),
                       reinterpret_cast<const uint32_t *>(zeros), N, K, group, fmt, slices, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quant_error_final_kernel, dim3(1), dim3(kQeThreads), 0, stream, partial, blocks,
                       (double)N * (double)K, out);
    return hipGetLastError();
}

hipError_t launch_scale_activations(const void *x, bool bf16, const float *act_mul, void *x_out, int64_t M, int K,
                                    hipStream_t stream) {
    const int upr = K / 8;
    const int64_t units = M * upr;
    const dim3 grid((unsigned)ceil_div(units, 256));
    auto *xi = reinterpret_cast<const uint4 *>(x);
    auto *mi = reinterpret_cast<const float4 *>(act_mul);
    auto *xo = reinterpret_cast<uint4 *>(x_out);
    if (bf16)
        hipLaunchKernelGGL(scale_activations_kernel<true>, grid, dim3(256), 0, stream, xi, mi, xo, units, upr);
    else
        hipLaunchKernelGGL(scale_activations_kernel<false>, grid, dim3(256), 0, stream, xi, mi, xo, units, upr);
    return hipGetLastError();
}

}  // namespace w4a16
