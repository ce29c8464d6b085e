// Decode GEMV host side: launch plan, LDS sizing and the dispatch over the
// weight formats. The kernel is in gemv_kernel.hpp; each weight format is
// compiled in its own translation unit (this one: the 4-bit zero-point
// format; gemv_sym4.hip, gemv_sym8.hip).
#include "gemv_kernel.hpp"

namespace w4a16 {

int gemv_xcols(int64_t K, int waves) {
    const int64_t T = ceil_div(K / kChunk, kColChunks);
    return (int)ceil_div(T, waves);
}

size_t gemv_lds_bytes(int64_t M, int64_t K, bool bf16, int waves, int fmt) {
    return wave_lds_bytes((int)M, gemv_xcols(K, waves), bf16 || fmt == kKq4) * waves;
}

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int32_t group) {
    (void)M;
    (void)group;
    static const int forced_waves = [] {
        const char *v = getenv("W4A16_GEMV_WAVES");
        return v ? atoi(v) : 0;
    }();
    GemvPlan p{};
    p.row_blocks = (int)ceil_div(N, kGemvRowsPerWg);
    const int64_t columns = ceil_div(K / kChunk, kColChunks);
    // four waves per workgroup measured best for the decode shapes, also for
    // K = 28672 (56 columns per wave); more only for still longer K, never
    // more waves than columns
    int64_t w = 4;
    if (columns > 4 * 64) w = ceil_div(columns, 64);
    if (w > columns) w = columns;
    if (forced_waves > 0) w = forced_waves;
    if (w > kMaxWaves) w = kMaxWaves;
    if (w < 1) w = 1;
    p.waves = (int)w;
    return p;
}

hipError_t launch_gemv(const void *x, bool bf16, const void *qweight, const void *scales,
                       const void *zeros, void *y, int M, int N, int K, int group, int fmt,
                       const float *act_mul, const GemvPlan &plan, hipStream_t stream) {
    const float *am = act_mul;
    switch (fmt) {
        case kSym4: return launch_gemv_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, am, plan, stream);
        case kSym8: return launch_gemv_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, am, plan, stream);
        case kKq4: return launch_gemv_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, am, plan, stream);
        default: return launch_gemv_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, am, plan, stream);
    }
}

template hipError_t launch_gemv_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                            int, int, int, int, const float *, const GemvPlan &, hipStream_t);

}  // namespace w4a16
