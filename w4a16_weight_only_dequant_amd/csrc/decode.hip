// Decode kernel, host side: launch plan and the dispatch over the weight
// formats. The kernel is in decode_kernel.hpp; each weight format is compiled
// in its own translation unit (this one: the 4-bit zero-point format;
// decode_sym4.hip, decode_sym8.hip, decode_kq4.hip).
#include "decode_kernel.hpp"

namespace w4a16 {

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int32_t group, int fmt, bool awq) {
    (void)N;
    DecodePlan p{};
    p.ok = false;
    if (M < 1 || M > kDecodeMaxM || K <= 0) return p;
    const int64_t T = ceil_div(K / kChunk, kColChunks);   // 128-weight columns of K
    const int mt = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8));
    // eight columns per wave while that fits the workgroup; sixteen (one or
    // two activation rows, no AWQ: their registers) for K up to 32768
    int ncol;
    if (ceil_div(T, 8) <= kDecMaxWaves) ncol = 8;
    else if (mt <= 2 && !awq && ceil_div(T, 16) <= kDecMaxWaves) ncol = 16;
    else return p;
    p.mt = mt;
    p.ncol = ncol;
    p.waves = (int)ceil_div(T, ncol);
    p.lds = (size_t)p.waves * (size_t)dec_lds(mt, ncol, fmt == kKq4 ? 256 : group, fmt).total;
    p.ok = true;
    return p;
}

hipError_t launch_decode(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                         void *y, int M, int N, int K, int group, int fmt, const float *act_mul,
                         const DecodePlan &plan, hipStream_t stream) {
    switch (fmt) {
        case kSym4: return launch_decode_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, stream);
        case kSym8: return launch_decode_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, stream);
        case kKq4: return launch_decode_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, stream);
        default: return launch_decode_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, stream);
    }
}

template hipError_t launch_decode_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                              int, int, int, int, const float *, const DecodePlan &, hipStream_t);

}  // namespace w4a16
